#!/usr/bin/env python3
"""Benchmark of the DLRMv1 forward hot path on one MI355X.

Default workload: the fused multi-table EmbeddingBag(sum) gather + strict-
lower-triangle pairwise-dot interaction at B=2048, K=32 tables x 1,000,000
rows x D=64, 20 Zipf(1.05) indices per bag (dlrm_emb_interact, one launch).

A step is one pass of that hot path over one batch.  Steps rotate through
several independently drawn index batches, and by default the caches are
flushed before each step (a 1 GiB read, outside the timed region: it evicts
L2 and the Infinity Cache without leaving dirty lines to write back), so the
table rows come from HBM as they would for a fresh batch; each step's kernel
time is taken with HIP events on the stream the kernel runs on.  `--warm`
skips the flush.

Prints ONE JSON line on stdout (progress goes to stderr):
  value         samples/s = B / mean event-timed step time
  ms_per_step   mean event-timed step time
  roofline      the fused kernel against MI355X's 8 TB/s HBM peak, with its
                own duration (events recorded by the launch itself, as
                rocprofv3 times the kernel).  `achieved` counts bytes that the
                memory side served: the copy-calibrated rocprofv3 FETCH_SIZE +
                WRITE_SIZE of profiles/counters.json when they were taken on
                the current kernel sources (`traffic`), else the compulsory
                bytes (each distinct row once + indices + dense + output);
                `byte_model` says which.  The logical bytes (every gathered
                row counted each time: the survey's algorithmic bytes) give
                `logical_gbps`, an L2-assisted rate that is not an HBM rate.
                `practical_peak_gbps` is the library's streaming-read kernel
                over 4 GiB.
  cpu_baseline  the CPU oracle timed on the host on the same workload

`extra` carries the warm step, the stacked-table layout, the gather and the
interaction as separate calls (`rows`), the same launch with uniform indices
(`uniform`, no hot rows), the host-inclusive call time, a plain device
copy's rate and the device properties the rooflines assume.

The JSON line also carries `variants`: the same fused launch with bfloat16
tables, FP8 tables, mean pooling, per-sample weights and CSR bags of size 0..40
(dlrm_emb_interact_pool), `cells`: the pages' small DLRMv1 cells (nc x
batch) per call, eager dlrm_forward against a graph-replayed plan, and
`forward`: the full DLRMv1 forward at B=8192
(dlrm_forward), with each MLP layer timed alone against the f32 MFMA peak
(or HBM for the layers below the ridge point).

Options: --workload {nc32,nc32-uniform,mid,tiny,large,large-uniform} (or one variant,
nc32-bf16 / nc32-fp8 / nc32-mean / nc32-weighted / nc32-csr, timed alone), --no-variants,
--no-cells, --sweep (batch x num_tables grid instead of the default line),
--sweep-forward (the full forward over batch size), --warm, --no-cpu-baseline,
--no-forward; for profiler runs: --profile-run (the timed cold steps only),
--profile-forward B1,B2 (cold full forwards), --profile-linear N K LDA (one
layer), --forward-penalty (the B=8192 forward's MLP launches in and out of
the forward), --read-probe (1 GiB streaming reads, the practical peak and the
FETCH_SIZE scale), --copy-calibration (1 GiB copies, the WRITE_SIZE scale);
--record-counters DIR (counter runs to profiles/counters.json).
"""
import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
F32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense f32 matrix, published
METRIC = ("samples/sec + µs/forward (emb-bag+interact, B=2048 nc=32); "
          "achieved HBM GB/s")
COUNTERS_JSON = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = ["dlrm_embedding_bag_amd/csrc/emb_interact.hip",
                  "dlrm_embedding_bag_amd/csrc/gather_interact.hpp",
                  "dlrm_embedding_bag_amd/csrc/common.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ byte models --
def emb_interact_bytes_per_sample(K, D, L):
    """Algorithmic bytes of the fused gather + interaction for one sample:
    gathered rows K*L*D*4 + indices K*L*4 + dense D*4 + output (D+P)*4."""
    F = K + 1
    P = F * (F - 1) // 2
    return K * L * D * 4 + K * L * 4 + D * 4 + (D + P) * 4


def pool_bytes_per_sample(w, K, n_idx_per_sample):
    """Algorithmic bytes of the fused gather + interaction of a general bag
    form for one sample: gathered rows (row bytes by storage type) + indices
    + per-sample weights + CSR offsets + dense + output."""
    F = K + 1
    P = F * (F - 1) // 2
    row = w.dim * {"f32": 4, "bf16": 2, "fp8": 1}[w.table_dtype]
    return (n_idx_per_sample * (row + 4 + (4 if w.weighted else 0))
            + (K * 4 if w.lengths != "fixed" else 0) + w.dim * 4 + (w.dim + P) * 4)


# ------------------------------------------------------------- workloads --
class PoolCase:
    """Device inputs for dlrm_emb_interact_pool (bf16 tables, mean pooling,
    per-sample weights, CSR bags) plus prepared C-ABI arguments."""

    def __init__(self, w, nbatches, seed, stream):
        import torch
        from dlrm_embedding_bag_amd import abi, inputs
        self.w = w
        self.B, self.K, self.D = w.batch, w.num_tables, w.dim
        self.tables = [inputs.table_device_typed(w, k, seed) for k in range(self.K)]
        self.lib = abi.load()
        self.stream = stream
        self.batches = []
        self.n_idx = 0
        for nb in range(nbatches):
            sd = seed + 7919 * nb
            idx = [inputs.indices(w, k, sd) for k in range(self.K)]
            offs = ([torch.from_numpy(inputs.csr_offsets(w, k, sd)).cuda() for k in range(self.K)]
                    if w.lengths != "fixed" else None)
            wts = ([torch.from_numpy(inputs.sample_weights(w, k, idx[k].shape[0], sd)).cuda()
                    for k in range(self.K)] if w.weighted else None)
            idx_d = [torch.from_numpy(i).cuda() for i in idx]
            dense = torch.from_numpy(inputs.dense(w, sd)).cuda()
            # the interaction reads B dense rows of D floats
            if tuple(dense.shape) != (self.B, w.dim):
                raise ValueError(f"dense input {tuple(dense.shape)} is not (B, D) = "
                                 f"{(self.B, w.dim)}")
            F = self.K + 1
            out = torch.empty((self.B, w.dim + F * (F - 1) // 2), dtype=torch.float32,
                              device="cuda")
            sc = inputs.table_scale(w)
            g = abi._BagsArg(self.tables, idx_d, offs, wts, w.pool, self.B,
                             [sc] * self.K if sc else None)
            args = (ctypes.byref(g.struct), dense.data_ptr(), out.data_ptr(), None,
                    stream.cuda_stream)
            self.batches.append((g, dense, out, args))
            self.n_idx += sum(i.shape[0] for i in idx)
        self.n_idx /= nbatches

    def run(self, nb):
        rc = self.lib.dlrm_emb_interact_pool(*self.batches[nb % len(self.batches)][3])
        if rc != 0:
            raise RuntimeError(f"dlrm_emb_interact_pool failed with status {rc}")

    def bytes_per_launch(self):
        return self.B * pool_bytes_per_sample(self.w, self.K, self.n_idx / self.B)


class EmbInteractCase:
    """Device inputs for dlrm_emb_interact plus prepared C-ABI arguments."""

    def __init__(self, w, nbatches, seed, stream, batch=None, num_tables=None,
                 tables=None):
        import numpy as np
        import torch
        from dlrm_embedding_bag_amd import abi, inputs
        self.w = w
        self.B = batch or w.batch
        self.K = num_tables or w.num_tables
        self.D = w.dim
        self.L = w.bag
        if tables is None:
            if w.table_source == "device":
                tables = [inputs.table_device(w, k, seed) for k in range(self.K)]
            else:
                tables = [torch.from_numpy(inputs.table_host(w, k, seed)).cuda()
                          for k in range(self.K)]
        self.tables = tables[:self.K]
        self.lib = abi.load()
        self.stream = stream
        self.batches = []
        for nb in range(nbatches):
            idx = [torch.from_numpy(inputs.indices(w, k, seed + 7919 * nb, batch=self.B)).cuda()
                   for k in range(self.K)]
            dense = torch.from_numpy(inputs.dense(w, seed + 7919 * nb, batch=self.B)).cuda()
            # the interaction reads B dense rows of D floats
            if tuple(dense.shape) != (self.B, self.D):
                raise ValueError(f"dense input {tuple(dense.shape)} is not (B, D) = "
                                 f"{(self.B, self.D)}")
            out = torch.empty((self.B, self.D + self.P), dtype=torch.float32, device="cuda")
            args = (self.K, self.B, self.D, abi._ptr_array(self.tables),
                    abi._i64_array([t.shape[0] for t in self.tables]), abi._ptr_array(idx),
                    None, abi._i64_array([i.numel() for i in idx]), dense.data_ptr(),
                    out.data_ptr(), None, stream.cuda_stream)
            self.batches.append((idx, dense, out, args))
        self.np = np

    @property
    def P(self):
        F = self.K + 1
        return F * (F - 1) // 2

    def run(self, nb):
        rc = self.lib.dlrm_emb_interact(*self.batches[nb % len(self.batches)][3])
        if rc != 0:
            raise RuntimeError(f"dlrm_emb_interact failed with status {rc}")

    def bytes_per_launch(self):
        return self.B * emb_interact_bytes_per_sample(self.K, self.D, self.L)

    def distinct_rows_fraction(self):
        """Distinct (table, row) pairs per gathered row, averaged over the
        rotating index batches."""
        fr = []
        for idx, *_ in self.batches:
            n = sum(int(i.unique().numel()) for i in idx)
            fr.append(n / (self.B * self.K * self.L))
        return statistics.mean(fr)

    def compulsory_bytes_per_launch(self, distinct_fraction):
        """What HBM must deliver at least with cold caches: every distinct row
        once, plus the indices, the dense input and the output."""
        rows = distinct_fraction * self.B * self.K * self.L * self.D * 4
        return int(rows + self.B * (self.K * self.L * 4 + self.D * 4 + (self.D + self.P) * 4))


def time_steps(case, steps, warmup, cold, flush_buf, stream):
    """Event-timed steps; returns (per-step ms list, wall seconds of the bracket)."""
    import torch
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):   # the flush is ordered before each step
        for s in range(warmup):
            if cold:
                flush_buf.max()
            case.run(s)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            if cold:
                flush_buf.max()
            evs[s][0].record(stream)
            case.run(warmup + s)
            evs[s][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in evs], wall


class KernelTimer:
    """HIP event pairs that the library's kernel launches record at the
    kernel's own start and end (dlrm_set_kernel_timing_events), so a pair's
    elapsed time is one kernel's execution, as rocprofv3's kernel trace
    reports it, without the dispatch gap that events recorded around a call
    include.  The events come from the process's HIP runtime (the one torch
    loaded; the library links the same soname)."""

    def __init__(self, n):
        import torch
        from dlrm_embedding_bag_amd import abi
        torch.cuda.init()
        self.abi = abi
        self.hip = None
        for name in ("libamdhip64.so.7", "libamdhip64.so"):
            try:
                self.hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if self.hip is None:
            raise RuntimeError("the HIP runtime library is not loadable")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []
        for _ in range(n):
            pair = (ctypes.c_void_p(), ctypes.c_void_p())
            for e in pair:
                if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                    raise RuntimeError("hipEventCreate failed")
            self.events.append(pair)

    def arm(self, i):
        self.abi.dlrm_set_kernel_timing_events(self.events[i][0].value, self.events[i][1].value)

    def disarm(self):
        self.abi.dlrm_set_kernel_timing_events(None, None)

    def elapsed_ms(self, i):
        a, b = self.events[i]
        ms = ctypes.c_float()
        if (self.hip.hipEventSynchronize(b) != 0
                or self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0):
            raise RuntimeError("kernel timing events were not recorded")
        return ms.value

    def close(self):
        self.disarm()
        for pair in self.events:
            for e in pair:
                self.hip.hipEventDestroy(e)
        self.events = []


def time_kernel(case, steps, warmup, cold, flush_buf, stream):
    """Per-step kernel execution times (ms) of a one-launch case, from events
    the launch itself records (KernelTimer); the same flush and batch
    rotation as time_steps."""
    import torch
    timer = KernelTimer(steps)
    try:
        with torch.cuda.stream(stream):
            for s in range(warmup):
                if cold:
                    flush_buf.max()
                case.run(s)
            torch.cuda.synchronize()
            for s in range(steps):
                if cold:
                    flush_buf.max()
                timer.arm(s)
                case.run(warmup + s)
                timer.disarm()
            torch.cuda.synchronize()
        return [timer.elapsed_ms(s) for s in range(steps)]
    finally:
        timer.close()


# ----------------------------------------------------------- CPU baseline --
def cpu_baseline(case, max_seconds=20.0):
    """The CPU oracle on this workload: the full batch (fewer samples if one
    pass would exceed max_seconds), tables copied to the host, single-threaded
    C with fp64 sums, repeated until about 10 s of CPU time; the median run."""
    import numpy as np
    import oracle
    idx, dense, out, _ = case.batches[0]
    log("cpu_baseline: copying tables to the host ...")
    tables = [t.cpu().numpy() for t in case.tables]
    idx_h = [i.cpu().numpy() for i in idx]
    dense_h = dense.cpu().numpy()
    B = case.B
    # sample size: the whole batch, unless one pass would exceed the bound
    samples = B
    t0 = time.perf_counter()
    probe = max(1, min(B, 64))
    oracle.interact(dense_h[:probe], oracle.emb_bag_sum(
        tables, [x[:probe * case.L] for x in idx_h], batch=probe))
    est = (time.perf_counter() - t0) / probe * B
    if est > max_seconds:
        samples = max(1, int(B * max_seconds / est))
    idx_s = [x[:samples * case.L] for x in idx_h]
    runs = []
    # one thread, pinned to one core for the timed runs
    prev = os.sched_getaffinity(0)
    core = min(prev)
    os.sched_setaffinity(0, {core})
    try:
        while True:
            t0 = time.perf_counter()
            E = oracle.emb_bag_sum(tables, idx_s, batch=samples)
            R = oracle.interact(dense_h[:samples], E)
            runs.append(time.perf_counter() - t0)
            if sum(runs) >= 10.0:   # about 10 s of CPU work in all
                break
    finally:
        os.sched_setaffinity(0, prev)
    t = statistics.median(runs)
    got = out.cpu().numpy()[:samples]
    err = float(np.abs(got - R).max())
    return {"value": samples / t, "unit": "samples/s", "cores": 1, "kind": "oracle",
            "sample": f"{samples} of {B} samples of the same batch, full tables in host "
                      f"memory, single-threaded C oracle (fp64 sums) pinned to core {core} "
                      f"of {len(prev)} available, median of {len(runs)} run(s) of {t:.3f} s",
            "max_abs_diff_vs_gpu": err}


def forward_cpu_baseline(w, tables_dev, idx_host, dense_host, bottom, top, out_gpu,
                         max_seconds=20.0, seed=0):
    """The CPU oracle's whole DLRMv1 forward (oracle.forward: fp64 sums,
    single-threaded C, pinned to one core) on a bounded prefix of the same
    batch.  The sample's tables are cut down to the rows its bags touch
    (indices renumbered), which leaves every pooled sum unchanged and keeps
    host memory small; repeated until ~10 s of CPU work, median run; also the
    largest difference from the GPU forward on those samples."""
    import numpy as np
    import torch
    import oracle
    B, L = w.batch, w.bag

    def cut(samples):
        subs, sidx = [], []
        for t, idx in zip(tables_dev, idx_host):
            bags = idx[:samples * L]
            rows = np.unique(bags)
            subs.append(t.index_select(0, torch.from_numpy(rows.astype(np.int64)).to(t.device))
                        .cpu().numpy())
            sidx.append(np.searchsorted(rows, bags).astype(np.int32))
        return subs, sidx

    probe = 64
    subs, sidx = cut(probe)
    t0 = time.perf_counter()
    oracle.forward(dense_host[:probe], bottom, top, subs, sidx)
    per = (time.perf_counter() - t0) / probe
    samples = min(B, max(probe, int(max_seconds / per)))
    subs, sidx = cut(samples)
    prev = os.sched_getaffinity(0)
    core = min(prev)
    os.sched_setaffinity(0, {core})
    runs = []
    try:
        while True:
            t0 = time.perf_counter()
            want, _, _ = oracle.forward(dense_host[:samples], bottom, top, subs, sidx)
            runs.append(time.perf_counter() - t0)
            if sum(runs) >= 10.0:
                break
    finally:
        os.sched_setaffinity(0, prev)
    t = statistics.median(runs)
    got = out_gpu[:samples]
    err = float(np.abs(got - want).max())
    ok = bool(np.all(np.abs(got - want) <= 1e-5 + 1e-5 * np.abs(want)))
    log(f"forward cpu baseline: {samples / t:.0f} samples/s on one core ({samples} samples), "
        f"max abs diff vs GPU {err:.2e}")
    return {"value": samples / t, "unit": "samples/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {samples} of {B} samples of the same forward batch (tables cut "
                      f"to the rows their bags touch), single-threaded C oracle (fp64 sums) "
                      f"pinned to core {core} of {len(prev)} available, median of {len(runs)} "
                      f"run(s) of {t:.3f} s",
            "max_abs_diff_vs_gpu": err, "within_tolerance": ok}


def read_traffic(kernel_hash, workload):
    """The committed counter record of `workload` (profiles/counters.json)
    if it was taken on the current kernel sources, else None."""
    try:
        with open(COUNTERS_JSON) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    entry = c.get(workload)
    if not entry or entry.get("kernel_source_hash") != kernel_hash:
        return None
    return entry


def hbm_roofline(logical_bytes, compulsory_bytes, kernel_ms, counters, practical):
    """The HBM roofline of one launch.  `achieved` holds bytes that HBM's side
    of the chip actually served: the copy-calibrated FETCH_SIZE + WRITE_SIZE
    of the committed counter run on the current kernel (L2-miss traffic; it
    also counts Infinity Cache hits, so it bounds DRAM traffic from above),
    else the compulsory bytes (every distinct row once + indices + dense +
    output, a lower bound with cold caches).  Either way frac <= 1 holds for a
    physical transfer.  The logical (algorithmic) bytes, which count repeated
    rows every time, are reported beside it as logical_gbps: repeated rows
    come from L2, so that rate is not an HBM rate."""
    t = kernel_ms * 1e-3
    measured = counters.get("hbm_bytes_per_launch") if counters else None
    if measured:
        hbm, model = measured, ("memory-side bytes per launch measured by rocprofv3 "
                                "(FETCH_SIZE + WRITE_SIZE, scaled by a known-size read and "
                                "copy; L2 misses, Infinity Cache hits included)")
    else:
        hbm, model = compulsory_bytes, ("compulsory bytes per launch (distinct rows once + "
                                        "indices + dense + output; no counter run matches "
                                        "the current kernel)")
    r = {"bound": "hbm", "achieved": hbm / t / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": hbm / t / 1e9 / HBM_PEAK_GBPS, "traffic": measured,
         "byte_model": model, "bytes_per_launch": hbm,
         "logical_bytes_per_launch": logical_bytes,
         "logical_gbps": logical_bytes / t / 1e9,
         "compulsory_bytes_per_launch": compulsory_bytes,
         "compulsory_gbps": compulsory_bytes / t / 1e9,
         "compulsory_frac": compulsory_bytes / t / 1e9 / HBM_PEAK_GBPS}
    if counters and counters.get("dram_bytes_per_launch"):
        r["dram_counter_bytes_per_launch"] = counters["dram_bytes_per_launch"]
        r["dram_counter_gbps"] = counters["dram_bytes_per_launch"] / t / 1e9
    if practical:
        r["practical_peak_gbps"] = practical["gbps"]
        r["frac_of_practical_peak"] = r["achieved"] / practical["gbps"]
        r["practical_peak"] = practical
    return r


def practical_read_peak(stream, gib=4, reps=10):
    """Read rate of the library's streaming-read kernel (dlrm_stream_read)
    over a buffer far larger than the Infinity Cache: kernel time from
    launch-recorded events, median of `reps` launches."""
    import torch
    from dlrm_embedding_bag_amd import abi
    buf = torch.zeros(gib << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, device="cuda")
    nbytes = buf.numel() * 4
    timer = KernelTimer(reps)
    try:
        with torch.cuda.stream(stream):
            abi.dlrm_stream_read(buf, sink, stream=stream)
            for i in range(reps):
                timer.arm(i)
                abi.dlrm_stream_read(buf, sink, stream=stream)
                timer.disarm()
        torch.cuda.synchronize()
        ms = statistics.median(timer.elapsed_ms(i) for i in range(reps))
    finally:
        timer.close()
    del buf
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"practical peak: the streaming-read kernel reads {gib} GiB at {gbps:.0f} GB/s "
        f"({gbps / HBM_PEAK_GBPS:.3f} of 8 TB/s)")
    return {"gbps": gbps, "bytes": nbytes, "kernel_ms": ms, "frac_of_spec": gbps / HBM_PEAK_GBPS,
            "kernel": "dlrm_stream_read (stream_read_kernel): 16-byte loads, 8 in flight per "
                      "lane, 2048 workgroups of 256 lanes, median of 10 launches"}


# ------------------------------------------------------------------ main --
def bench_emb_interact(args, stream):
    import torch
    from dlrm_embedding_bag_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    log(f"workload {w.name}: {w.description}")
    t0 = time.perf_counter()
    case = EmbInteractCase(w, args.batches, args.seed, stream)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    flush = torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda")
    cold = not args.warm
    times, wall = time_steps(case, args.steps, args.warmup, cold, flush, stream)
    ms = statistics.mean(times)
    med = statistics.median(times)
    log(f"{'cold' if cold else 'warm'} step: mean {ms * 1000:.1f} us, median "
        f"{med * 1000:.1f} us over {args.steps} steps")
    nbytes = case.bytes_per_launch()
    # the roofline takes the kernel's own duration (events recorded by the
    # launch), which is what rocprofv3's kernel trace reports for it
    ktimes = time_kernel(case, args.steps, args.warmup, cold, flush, stream)
    kms = statistics.mean(ktimes)
    log(f"kernel alone: mean {kms * 1000:.1f} us, median "
        f"{statistics.median(ktimes) * 1000:.1f} us over {args.steps} steps")
    practical = practical_read_peak(stream) if not args.profile_run else None
    extra = {"median_ms_per_step": med, "min_ms_per_step": min(times),
             "wall_ms_per_step_incl_flush": wall / args.steps * 1e3,
             "distinct_row_fraction": case.distinct_rows_fraction()}
    if cold and not args.profile_run:
        wt, _ = time_steps(case, args.steps, 2, False, flush, stream)
        wms = statistics.mean(wt)
        extra["warm_ms_per_step"] = wms
        extra["warm_samples_per_s"] = case.B / (wms * 1e-3)
        extra["warm_logical_gbps"] = nbytes / (wms * 1e-3) / 1e9
        log(f"warm step: mean {wms * 1000:.1f} us")
    # the same batch with the K tables carved out of one allocation (stacked
    # layout): table k = base + row_offsets[k] * D, nothing else changes
    if not args.profile_run:
        import torch
        stack = torch.empty((case.K * w.rows, case.D), device="cuda")
        for k, t in enumerate(case.tables):
            stack[k * w.rows:(k + 1) * w.rows] = t
        scase = EmbInteractCase(w, args.batches, args.seed, stream,
                                tables=[stack[k * w.rows:(k + 1) * w.rows] for k in range(case.K)])
        st, _ = time_steps(scase, args.steps, args.warmup, cold, flush, stream)
        extra["stacked_layout_ms_per_step"] = statistics.mean(st)
        log(f"stacked layout: mean {statistics.mean(st) * 1000:.1f} us")
        del scase, stack
    if not args.profile_run:
        res_rows = bench_rows(case, args, stream, flush, cold)
        extra["rows"] = res_rows
    if not args.profile_run and w.name == "nc32":
        extra["uniform"] = bench_uniform(case, args, stream, flush, cold, practical)
    if not args.profile_run:
        extra["host_inclusive_us"] = host_inclusive_time(case, args.steps, cold, flush,
                                                         stream) * 1e3
    khash = kernel_source_hash()
    roofline = hbm_roofline(nbytes, case.compulsory_bytes_per_launch(
        extra["distinct_row_fraction"]), kms, read_traffic(khash, w.name), practical)
    roofline.update({"kernel": "interact_kernel (fused gather + interaction, dlrm_emb_interact)",
                     "kernel_us": kms * 1e3,
                     "timing": "kernel execution: events recorded by the launch itself "
                               "(hipExtLaunchKernel), mean over the timed cold steps",
                     "kernel_source_hash": khash})
    log(f"roofline: {roofline['achieved']:.0f} GB/s of {roofline['byte_model']} "
        f"(frac {roofline['frac']:.3f} of 8 TB/s); logical {roofline['logical_gbps']:.0f} GB/s")
    res = {"metric": METRIC, "value": case.B / (ms * 1e-3), "unit": "samples/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "us_per_forward": ms * 1e3, "achieved_hbm_gbps": roofline["achieved"],
           "step_logical_gbps": nbytes / (ms * 1e-3) / 1e9,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded N(0, 0.01^2) tables, Zipf/uniform int32 indices, "
                   "N(0,1) dense)",
           "config": {"workload": f"{w.name}: {w.description}", "batch": case.B,
                      "num_tables": case.K, "dim": case.D, "bag": case.L, "rows": w.rows,
                      "index_dist": w.dist, "cache": "cold" if cold else "warm",
                      "index_batches": args.batches},
           "roofline": roofline, "extra": extra}
    if not args.profile_run:
        extra["device"] = device_info()
        extra["copy_gbps"] = copy_rate(stream)
        log(f"a 1 GiB device copy moves {extra['copy_gbps']:.0f} GB/s (read + write)")
    if not args.no_cpu_baseline and not args.profile_run:
        res["cpu_baseline"] = cpu_baseline(case)
        log(f"cpu baseline: {res['cpu_baseline']['value']:.0f} samples/s")
    return res


def bench_rows(case, args, stream, flush, cold):
    """The gather and the interaction as separate calls on the benchmark batch
    (emb_bag_sum_multi to a (B, K, D) buffer, then dlrm_interact_lower_tri
    from it): each timed alone, with its algorithmic bytes, and checked equal
    to the fused call's output."""
    import torch
    B, K, D, L, P = case.B, case.K, case.D, case.L, case.P
    idx, dense, out, args0 = case.batches[0]
    lib = case.lib
    emb = torch.empty((B, K, D), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    gargs = (K, B, D, args0[3], args0[4], args0[5], None, args0[7], emb.data_ptr(),
             stream.cuda_stream)
    iargs = (B, K, D, dense.data_ptr(), emb.data_ptr(), out2.data_ptr(), stream.cuda_stream)

    def gather():
        rc = lib.emb_bag_sum_multi(*gargs)
        if rc:
            raise RuntimeError(f"emb_bag_sum_multi: {rc}")

    def interact():
        rc = lib.dlrm_interact_lower_tri(*iargs)
        if rc:
            raise RuntimeError(f"dlrm_interact_lower_tri: {rc}")

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        case.run(0)
        gather()
        interact()
    torch.cuda.synchronize()
    same = bool(torch.equal(out2, out))
    t_g = _event_time(gather, stream, args.steps, args.warmup, cold, flush)
    t_i = _event_time(interact, stream, args.steps, args.warmup, cold, flush)
    t_u = _event_time(lambda: (gather(), interact()), stream, args.steps, args.warmup, cold,
                      flush)
    # the gather's logical bytes count every repeated row; its compulsory
    # bytes count each distinct row once (plus indices and the output)
    g_bytes = B * K * L * (D + 1) * 4 + B * K * D * 4
    distinct = sum(int(i.unique().numel()) for i in idx)
    g_comp = distinct * D * 4 + B * K * L * 4 + B * K * D * 4
    # the interaction reads each pooled vector and dense row once: no reuse
    i_bytes = B * K * D * 4 + B * D * 4 + B * (D + P) * 4
    rows = {"cache": "cold" if cold else "warm",
            "emb_bag_sum_multi": {"us": t_g * 1e3, "logical_bytes": g_bytes,
                                  "logical_gbps": g_bytes / (t_g * 1e-3) / 1e9,
                                  "compulsory_bytes": g_comp,
                                  "compulsory_gbps": g_comp / (t_g * 1e-3) / 1e9,
                                  "compulsory_frac": g_comp / (t_g * 1e-3) / 1e9 / HBM_PEAK_GBPS},
            "dlrm_interact_lower_tri": {"us": t_i * 1e3, "bytes": i_bytes,
                                        "gbps": i_bytes / (t_i * 1e-3) / 1e9,
                                        "frac": i_bytes / (t_i * 1e-3) / 1e9 / HBM_PEAK_GBPS},
            "unfused_pair_us": t_u * 1e3,
            "unfused_equals_fused": same}
    log(f"rows: gather alone {t_g * 1e3:.1f} us ({rows['emb_bag_sum_multi']['logical_gbps']:.0f} "
        f"GB/s logical), interaction alone {t_i * 1e3:.1f} us "
        f"({rows['dlrm_interact_lower_tri']['gbps']:.0f} GB/s), both {t_u * 1e3:.1f} us; "
        f"equal to fused: {same}")
    del emb, out2
    return rows


def bench_variant_line(args, stream):
    """One variant workload alone (--workload nc32-bf16 etc.): its cold
    timed steps only, for profiler runs of the variant kernels."""
    import torch
    from dlrm_embedding_bag_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    log(f"workload {w.name}: {w.description}")
    case = PoolCase(w, args.batches, args.seed, stream)
    flush = torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda")
    times, _ = time_steps(case, args.steps, args.warmup, not args.warm, flush, stream)
    ms = statistics.mean(times)
    kms = statistics.mean(time_kernel(case, args.steps, args.warmup, not args.warm, flush,
                                      stream))
    nbytes = case.bytes_per_launch()
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"{w.name}: mean {ms * 1000:.1f} us, {gbs:.0f} GB/s; kernel alone {kms * 1000:.1f} us")
    return {"workload": f"{w.name}: {w.description}", "ms_per_step": ms,
            "samples_per_s": case.B / (ms * 1e-3), "logical_gbps": gbs,
            "kernel_us": kms * 1e3,
            "kernel_logical_gbps": nbytes / (kms * 1e-3) / 1e9, "steps": args.steps}


def _event_time(fn, stream, steps, warmup, cold, flush):
    """Median event time (ms) of fn() on `stream`, caches flushed before each
    call when cold."""
    import torch
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            if cold:
                flush.max()
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for s in range(steps):
            if cold:
                flush.max()
            evs[s][0].record(stream)
            fn()
            evs[s][1].record(stream)
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in evs)


def _back_to_back_time(fn, stream, launches=50, rounds=5):
    """Per-launch time (ms) of `launches` consecutive fn() calls between two
    events, median over rounds: the kernel's steady-state duration, as a
    kernel trace reports it, without the per-launch event overhead."""
    import torch
    torch.cuda.synchronize()
    per = []
    with torch.cuda.stream(stream):
        for _ in range(3):
            fn()
        for _ in range(rounds):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(launches):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / launches)
    return statistics.median(per)


def bench_forward(args, stream, flush):
    """The full DLRMv1 forward (dlrm_forward, one C call, 7 launches) at
    B=8192, with each MLP layer and the gather + interaction also timed alone
    against its roofline."""
    import torch
    from dlrm_embedding_bag_amd import abi, inputs
    w = inputs.WORKLOADS["dlrm"]
    log(f"forward workload: {w.description}")
    tables = [inputs.table_device(w, k, args.seed) for k in range(w.num_tables)]
    idx = [torch.from_numpy(inputs.indices(w, k, args.seed)).cuda() for k in range(w.num_tables)]
    dense_in = torch.from_numpy(inputs.dense(w, args.seed)).cuda()
    bottom, top = inputs.dlrm_layers(w, args.seed)
    dev = lambda a: torch.from_numpy(a).cuda()
    bl = [(dev(a), dev(b), act) for a, b, act in bottom]
    tl = [(dev(a), dev(b), act) for a, b, act in top]
    model = abi.DlrmModel(bl, tl, tables)
    B = w.batch
    ws = torch.empty(model.workspace_bytes(B), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, 1), device="cuda")
    lib = abi.load()
    fwd_args = (ctypes.byref(model.struct), B, dense_in.data_ptr(), abi._ptr_array(idx), None,
                abi._i64_array([i.numel() for i in idx]), out.data_ptr(), ws.data_ptr(),
                ws.numel(), stream.cuda_stream)
    torch.cuda.synchronize()

    def fwd():
        rc = lib.dlrm_forward(*fwd_args)
        if rc != 0:
            raise RuntimeError(f"dlrm_forward failed with status {rc}")
    cold = not args.warm
    t_fwd = _event_time(fwd, stream, args.steps, args.warmup, cold, flush)
    log(f"forward: {t_fwd * 1000:.1f} us ({'cold' if cold else 'warm'})")
    cpu = None
    if not args.no_cpu_baseline:
        with torch.cuda.stream(stream):
            fwd()
        torch.cuda.synchronize()
        cpu = forward_cpu_baseline(w, tables, [inputs.indices(w, k, args.seed)
                                               for k in range(w.num_tables)],
                                   inputs.dense(w, args.seed), bottom, top,
                                   out.cpu().numpy())
    plan = abi.DlrmPlan(model, dense_in, idx, out=torch.empty((B, 1), device="cuda"),
                        workspace=torch.empty_like(ws), mode="graph")
    t_plan = _event_time(lambda: plan.run(stream), stream, args.steps, args.warmup, cold, flush)
    plan_same = bool(torch.equal(plan.out, out))
    plan.close()
    log(f"forward as a graph-mode plan: {t_plan * 1000:.1f} us, same output: {plan_same}")
    # each layer alone (warm: weights and activations are on-chip-sized), on
    # the forward's own activations: the bottom MLP on dense_in, the top MLP
    # on R = [d | dots] of this batch (a layer's time depends on its data: the
    # 415 -> 512 layer on N(0, 1) inputs and N(0, 0.05^2) weights takes ~10%
    # longer than on these)
    layers = []
    x = dense_in
    specs = [("bottom", i, l) for i, l in enumerate(bl)] + [("top", i, l) for i, l in enumerate(tl)]
    R = None
    acts = {}
    for part, i, (wt, b, act) in specs:
        if part == "top" and i == 0:
            R = abi.dlrm_emb_interact(tables, idx, x, stream=stream)
            x = R
        acts[(part, i)] = x
        n, k = wt.shape
        y = torch.empty((B, n), device="cuda")
        largs = (B, n, k, x.data_ptr(), x.stride(0), wt.data_ptr(), b.data_ptr(),
                 abi.ACTS[act], y.data_ptr(), n, stream.cuda_stream)
        t_one = _event_time(lambda: lib.linear_bias_act(*largs), stream, args.steps, 3, False,
                            flush)
        t = _back_to_back_time(lambda: lib.linear_bias_act(*largs), stream)
        flops = 2.0 * B * n * k
        nbytes = 4.0 * (B * k + n * k + n + B * n)
        tf = flops / (t * 1e-3) / 1e12
        gbs = nbytes / (t * 1e-3) / 1e9
        ai = flops / nbytes
        mfma_bound = ai > F32_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
        # "us": kernel duration from back-to-back launches; "us_isolated": one
        # launch between two events (adds the event and launch overhead)
        layers.append({"layer": f"{part}{i}: {k}->{n} {act}", "k": k, "n": n, "us": t * 1e3,
                       "us_isolated": t_one * 1e3, "tflops": tf,
                       "gbps": gbs, "bound": "mfma" if mfma_bound else "hbm",
                       "frac": (tf / F32_MFMA_PEAK_TFLOPS) if mfma_bound else gbs / HBM_PEAK_GBPS})
        x = y
    # the last two top layers as dlrm_forward runs them: one launch with the
    # sigmoid head folded into the 512 -> 256 layer's epilogue
    (w1, b1, a1), (wh, bh, ah) = tl[-2], tl[-1]
    n1, k1 = w1.shape
    xin = acts[("top", len(tl) - 2)]
    yh = torch.empty((B, 1), device="cuda")
    hargs = (B, n1, k1, xin.data_ptr(), xin.stride(0), w1.data_ptr(), b1.data_ptr(), abi.ACTS[a1],
             wh.data_ptr(), bh.data_ptr(), abi.ACTS[ah], yh.data_ptr(), 1, stream.cuda_stream)
    t_head = _back_to_back_time(lambda: lib.linear_bias_act_head(*hargs), stream)
    f_head = 2.0 * B * n1 * k1 + 2.0 * B * n1
    head = {"layer": f"top{len(tl) - 2}+head: {k1}->{n1} {a1}, {n1}->1 {ah} (one launch)",
            "us": t_head * 1e3, "tflops": f_head / (t_head * 1e-3) / 1e12,
            "frac": f_head / (t_head * 1e-3) / 1e12 / F32_MFMA_PEAK_TFLOPS}
    log(f"  {head['layer']:28s} {head['us']:7.1f} us {head['tflops']:6.1f} TFLOP/s "
        f"(frac {head['frac']:.2f})")
    # each MLP as one launch through the mlp_forward entry point (the fused
    # bottom-MLP kernel for the 13-512-256-64 stack, the chain kernel else)
    chains = []
    for part, spec, x_in, width_in in (("bottom", bl, dense_in, w.dense_in),
                                       ("top", tl, R, w.out_width)):
        arr = abi._layer_array(spec, part, [])
        n_out = spec[-1][0].shape[0]
        y = torch.empty((B, n_out), device="cuda")
        cargs = (B, len(spec), arr, x_in.data_ptr(), x_in.stride(0), y.data_ptr(), n_out,
                 stream.cuda_stream)
        if lib.mlp_forward(*cargs) != 0:
            continue
        t = _back_to_back_time(lambda: lib.mlp_forward(*cargs), stream)
        t_one = _event_time(lambda: lib.mlp_forward(*cargs), stream, args.steps, 3, False, flush)
        flops = sum(2.0 * B * wt.shape[0] * wt.shape[1] for wt, _, _ in spec)
        tf = flops / (t * 1e-3) / 1e12
        chains.append({"mlp": f"{part}: " + "-".join(str(v) for v in
                                                      [width_in] + [wt.shape[0] for wt, _, _ in spec]),
                       "us": t * 1e3, "us_isolated": t_one * 1e3, "tflops": tf,
                       "frac": tf / F32_MFMA_PEAK_TFLOPS})
        log(f"  fused {chains[-1]['mlp']:24s} {t * 1000:7.1f} us {tf:6.1f} TFLOP/s "
            f"(frac {tf / F32_MFMA_PEAK_TFLOPS:.2f})")
    # the gather + interaction of this workload alone, cold
    ecase = EmbInteractCase(inputs.Workload("dlrm-emb", B, w.num_tables, w.rows, w.dim, w.bag,
                                            "zipf", table_source="device"),
                            1, args.seed, stream, tables=tables)
    torch.cuda.synchronize()
    t_emb = _event_time(lambda: ecase.run(0), stream, args.steps, args.warmup, cold, flush)
    emb_bytes = ecase.bytes_per_launch()
    emb_comp = ecase.compulsory_bytes_per_launch(ecase.distinct_rows_fraction())
    mlp_us = sum(l["us"] for l in layers)
    mlp_flops = sum(2.0 * B * l["k"] * l["n"] for l in layers)
    # the MLP launches dlrm_forward issues at this batch: the bottom MLP as one
    # launch (the fused bottom kernel, timed through mlp_forward), the top
    # layers but the last two alone, those two as one launch
    nb = len(bl)
    bottom_chain = next((c for c in chains if c["mlp"].startswith("bottom")), None)
    bottom_us = bottom_chain["us"] if bottom_chain else sum(l["us"] for l in layers[:nb])
    fwd_mlp_us = bottom_us + sum(l["us"] for l in layers[nb:-2]) + head["us"]
    for l in layers:
        log(f"  {l['layer']:28s} {l['us']:7.1f} us {l['tflops']:6.1f} TFLOP/s "
            f"{l['gbps']:6.0f} GB/s ({l['bound']}, frac {l['frac']:.2f}; "
            f"{l['us_isolated']:.1f} us as one isolated launch)")
    log(f"  emb+interact {t_emb * 1000:.1f} us, {emb_bytes / (t_emb * 1e-3) / 1e9:.0f} GB/s "
        f"logical, {emb_comp / (t_emb * 1e-3) / 1e9:.0f} GB/s of compulsory bytes")
    return {"workload": f"dlrm: {w.description}", "batch": B, "cache": "cold" if cold else "warm",
            "us_per_forward": t_fwd * 1e3, "samples_per_s": B / (t_fwd * 1e-3),
            "cpu_baseline": cpu,
            "graph_plan_us_per_forward": t_plan * 1e3, "plan_equals_eager": plan_same,
            "emb_interact_us": t_emb * 1e3,
            "emb_interact_logical_gbps": emb_bytes / (t_emb * 1e-3) / 1e9,
            "emb_interact_compulsory_gbps": emb_comp / (t_emb * 1e-3) / 1e9,
            "emb_interact_compulsory_frac": emb_comp / (t_emb * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "mlp_chains": chains, "mlp_layers": layers, "mlp_head_fused": head,
            "mlp_layers_us_sum": mlp_us,
            "mlp_layers_tflops": mlp_flops / (mlp_us * 1e-6) / 1e12,
            "mlp_us_sum": fwd_mlp_us,
            "mlp_tflops": mlp_flops / (fwd_mlp_us * 1e-6) / 1e12,
            "mlp_frac_of_f32_mfma_peak": mlp_flops / (fwd_mlp_us * 1e-6) / 1e12
                                         / F32_MFMA_PEAK_TFLOPS,
            "mlp_timing": "each launch alone, warm, per launch of 50 back-to-back launches; "
                          "mlp_us_sum and the fraction cover the launches dlrm_forward issues "
                          "at this batch (the bottom MLP as one fused launch, the sigmoid "
                          "head folded into the layer before it), mlp_layers_* every layer "
                          "as its own launch"}


def bench_cells(args, stream):
    """The pages' small DLRMv1 cells (3 dense, D=16, L=2, 4096-row tables,
    MLPs 3-16 and (16+P)-16-1), nc x batch, warm: the whole forward per call
    through dlrm_forward (validation and packing each call, then the launch)
    and through plans (direct: the recorded launch; graph: a graph launch).  Each call is bracketed by events on the
    stream without synchronizing in between, so a host-bound call shows its
    host time; the pages' harness is mirrored (10 warmup, 5 rounds x 20
    calls, median of round medians)."""
    import torch
    from dlrm_embedding_bag_amd import abi, inputs
    lib = abi.load()
    cells = []
    for nc in (2, 4, 8, 16, 32):
        for b in (2, 16, 64, 256, 1024, 2048):
            w = inputs.cell_workload(nc, b)
            tables = [torch.from_numpy(inputs.table_host(w, k, args.seed)).cuda()
                      for k in range(nc)]
            bottom, top = inputs.dlrm_layers(w, args.seed)
            dv = lambda a: torch.from_numpy(a).cuda()
            model = abi.DlrmModel([(dv(a), dv(x), act) for a, x, act in bottom],
                                  [(dv(a), dv(x), act) for a, x, act in top], tables)
            idx = [dv(inputs.indices(w, k, args.seed)) for k in range(nc)]
            dense = dv(inputs.dense(w, args.seed))
            out = torch.empty((b, 1), device="cuda")
            ws = torch.empty(model.workspace_bytes(b), dtype=torch.uint8, device="cuda")
            fargs = (ctypes.byref(model.struct), b, dense.data_ptr(), abi._ptr_array(idx), None,
                     abi._i64_array([i.numel() for i in idx]), out.data_ptr(), ws.data_ptr(),
                     ws.numel(), stream.cuda_stream)
            plans = {m: abi.DlrmPlan(model, dense, idx, out=torch.empty((b, 1), device="cuda"),
                                     workspace=torch.empty_like(ws), mode=m)
                     for m in ("direct", "graph")}
            sptr = stream.cuda_stream

            def eager():
                lib.dlrm_forward(*fargs)
            fns = {"eager": eager}
            for m, pl in plans.items():
                fns[f"plan_{m}"] = (lambda h=pl._handle: lib.dlrm_plan_run(h, sptr))
            row = {"num_tables": nc, "batch": b}
            for name, fn in fns.items():
                row[f"{name}_us"] = _rounds_time(fn, stream) * 1e3
                row[f"{name}_host_us"] = _host_time(fn) * 1e3
            torch.cuda.synchronize()
            row["plans_equal_eager"] = all(bool(torch.equal(pl.out, out)) for pl in plans.values())
            cells.append(row)
            log(f"cell nc={nc:2d} b={b:5d}: eager {row['eager_us']:6.1f} us "
                f"(host {row['eager_host_us']:4.1f}), plan direct {row['plan_direct_us']:6.1f} us "
                f"(host {row['plan_direct_host_us']:4.1f}), plan graph {row['plan_graph_us']:6.1f} "
                f"us (host {row['plan_graph_host_us']:4.1f}); same output: "
                f"{row['plans_equal_eager']}")
            for pl in plans.values():
                pl.close()
            del model, tables, plans
    return {"model": "pages' cell: 3 dense, D=16, L=2, 4096-row tables, MLPs 3-16 and "
                     "(16+P)-16-1, uniform indices, warm",
            "timing": "events around each call, no sync between calls; 10 warmup, 5 rounds x 20 "
                      "calls, median of round medians",
            "cells": cells}


def _host_time(fn, calls=200):
    """Host time per call (ms): back-to-back calls without waiting for the
    GPU, the final synchronization excluded."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        fn()
    t = (time.perf_counter() - t0) / calls
    torch.cuda.synchronize()
    return t * 1e3


def _rounds_time(fn, stream, warmup=10, rounds=5, per_round=20):
    """Median of round medians of event-bracketed calls (ms)."""
    import torch
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
        meds = []
        for _ in range(rounds):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(per_round + 1)]
            evs[0].record(stream)
            for i in range(per_round):
                fn()
                evs[i + 1].record(stream)
            torch.cuda.synchronize()
            meds.append(statistics.median(evs[i].elapsed_time(evs[i + 1])
                                          for i in range(per_round)))
    return statistics.median(meds)


VARIANTS = ("nc32-bf16", "nc32-fp8", "nc32-mean", "nc32-weighted", "nc32-csr")


def bench_variants(args, stream, flush):
    """The fused gather + interaction of the general bag forms on the nc32
    shape (B=2048, K=32 x 1,000,000 x D=64, Zipf(1.05)): bfloat16 and FP8
    E4M3 tables, mean pooling, per-sample weights, CSR bags of size 0..40;
    cold, through dlrm_emb_interact_pool."""
    import torch
    from dlrm_embedding_bag_amd import inputs
    rows = []
    for name in VARIANTS:
        w = inputs.WORKLOADS[name]
        case = PoolCase(w, args.batches, args.seed, stream)
        torch.cuda.synchronize()
        times, _ = time_steps(case, args.steps, args.warmup, not args.warm, flush, stream)
        ms = statistics.mean(times)
        kms = statistics.mean(time_kernel(case, args.steps, 2, not args.warm, flush, stream))
        nbytes = case.bytes_per_launch()
        gbs = nbytes / (ms * 1e-3) / 1e9
        counters = read_traffic(kernel_source_hash(), name)
        row = {"workload": f"{name}: {w.description}", "us": ms * 1e3,
               "samples_per_s": case.B / (ms * 1e-3),
               "logical_bytes_per_launch": nbytes, "logical_gbps": gbs,
               "kernel_us": kms * 1e3,
               "kernel_logical_gbps": nbytes / (kms * 1e-3) / 1e9,
               "traffic": counters.get("hbm_bytes_per_launch") if counters else None}
        if row["traffic"]:
            row["traffic_gbps"] = row["traffic"] / (kms * 1e-3) / 1e9
            row["traffic_frac"] = row["traffic_gbps"] / HBM_PEAK_GBPS
        rows.append(row)
        log(f"variant {name:14s} {ms * 1000:7.1f} us {case.B / (ms * 1e-3) / 1e6:6.1f} M "
            f"samples/s {gbs:6.0f} GB/s")
        del case
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return rows


def bench_sweep(args, stream, flush):
    """batch x num_tables sweep of the fused gather + interaction (D=64,
    1,000,000 rows per table, 20 Zipf(1.05) indices per bag), cold."""
    import torch
    from dlrm_embedding_bag_amd import abi, inputs
    batches = [2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384]
    ntabs = [2, 4, 8, 16, 26, 32]
    base = inputs.WORKLOADS["nc32"]
    w = inputs.Workload("sweep", max(batches), max(ntabs), base.rows, base.dim, base.bag, "zipf",
                        table_source="device")
    tables = [inputs.table_device(w, k, args.seed) for k in range(w.num_tables)]
    idx = [torch.from_numpy(inputs.indices(w, k, args.seed)).cuda() for k in range(w.num_tables)]
    dense = torch.from_numpy(inputs.dense(w, args.seed)).cuda()
    lib = abi.load()
    cells = []
    for K in ntabs:
        for B in batches:
            F = K + 1
            P = F * (F - 1) // 2
            out = torch.empty((B, w.dim + P), device="cuda")
            xs = [i[: B * w.bag] for i in idx[:K]]
            a = (K, B, w.dim, abi._ptr_array(tables[:K]),
                 abi._i64_array([t.shape[0] for t in tables[:K]]), abi._ptr_array(xs), None,
                 abi._i64_array([x.numel() for x in xs]), dense.data_ptr(), out.data_ptr(), None,
                 stream.cuda_stream)
            t = _event_time(lambda: lib.dlrm_emb_interact(*a), stream, args.sweep_steps, 3,
                            not args.warm, flush)
            nbytes = B * emb_interact_bytes_per_sample(K, w.dim, w.bag)
            distinct = sum(int(x.unique().numel()) for x in xs)
            comp = distinct * w.dim * 4 + nbytes - B * K * w.bag * w.dim * 4
            gbs = nbytes / (t * 1e-3) / 1e9
            cgbs = comp / (t * 1e-3) / 1e9
            cells.append({"batch": B, "num_tables": K, "us": t * 1e3,
                          "samples_per_s": B / (t * 1e-3), "logical_gbps": gbs,
                          "distinct_row_fraction": distinct / (B * K * w.bag),
                          "compulsory_gbps": cgbs, "compulsory_frac": cgbs / HBM_PEAK_GBPS})
            log(f"sweep K={K:2d} B={B:5d}: {t * 1000:8.1f} us {gbs:7.0f} GB/s logical, "
                f"{cgbs:6.0f} GB/s compulsory")
    return {"dim": w.dim, "rows": w.rows, "bag": w.bag, "index_dist": "zipf(1.05)",
            "cache": "warm" if args.warm else "cold", "cells": cells}


def bench_sweep_forward(args, stream, flush):
    """Batch sweep of the full DLRMv1 forward (K=26 tables x 1,000,000 rows x
    D=64, 20 Zipf(1.05) indices per bag, MLPs 13-512-256-64 and
    415-512-256-1): the whole forward cold, the gather + interaction alone
    cold against the HBM roofline, and the six MLP layers alone (back to
    back, warm) against the f32 MFMA roofline."""
    import dataclasses
    import torch
    from dlrm_embedding_bag_amd import abi, inputs
    batches = [256, 1024, 2048, 4096, 8192, 16384]
    w = dataclasses.replace(inputs.WORKLOADS["dlrm"], batch=max(batches))
    tables = [inputs.table_device(w, k, args.seed) for k in range(w.num_tables)]
    idx = [torch.from_numpy(inputs.indices(w, k, args.seed)).cuda() for k in range(w.num_tables)]
    dense_in = torch.from_numpy(inputs.dense(w, args.seed)).cuda()
    bottom, top = inputs.dlrm_layers(w, args.seed)
    dev = lambda a: torch.from_numpy(a).cuda()
    bl = [(dev(a), dev(b), act) for a, b, act in bottom]
    tl = [(dev(a), dev(b), act) for a, b, act in top]
    model = abi.DlrmModel(bl, tl, tables)
    lib = abi.load()
    K, D, L = w.num_tables, w.dim, w.bag
    F = K + 1
    P = F * (F - 1) // 2
    cells = []
    for B in batches:
        xs = [i[: B * L] for i in idx]
        nidx = abi._i64_array([x.numel() for x in xs])
        ws = torch.empty(model.workspace_bytes(B), dtype=torch.uint8, device="cuda")
        out = torch.empty((B, 1), device="cuda")
        fa = (ctypes.byref(model.struct), B, dense_in.data_ptr(), abi._ptr_array(xs), None, nidx,
              out.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream)
        t_fwd = _event_time(lambda: lib.dlrm_forward(*fa), stream, args.sweep_steps, 3, True,
                            flush)
        d64 = torch.zeros((B, D), device="cuda")
        r = torch.empty((B, D + P), device="cuda")
        ea = (K, B, D, abi._ptr_array(tables), abi._i64_array([t.shape[0] for t in tables]),
              abi._ptr_array(xs), None, nidx, d64.data_ptr(), r.data_ptr(), None,
              stream.cuda_stream)
        t_emb = _event_time(lambda: lib.dlrm_emb_interact(*ea), stream, args.sweep_steps, 3,
                            True, flush)
        emb_bytes = B * emb_interact_bytes_per_sample(K, D, L)
        emb_comp = (sum(int(x.unique().numel()) for x in xs) * D * 4 + emb_bytes
                    - B * K * L * D * 4)
        # the six layers alone; at 7,137..8,192 samples also the MLP launches
        # dlrm_forward issues there (the bottom MLP as one launch and the
        # sigmoid head folded into the layer before it).  At other batches
        # the forward's MLP launches are the layers' own tiles, split over k
        # where the tiles leave CUs idle, and up to 1,024 samples a one-launch
        # bottom MLP whose output the interaction finishes: none of these is
        # callable alone, so only forward_us - emb_interact_us bounds them.
        mlp_t, mlp_f, t_by, acts = 0.0, 0.0, {}, {}
        x = dense_in[:B]
        for part, layers in (("bottom", bl), ("top", tl)):
            if part == "top":  # R = [d | dots] of this batch
                x = abi.dlrm_emb_interact(tables, xs, x, stream=stream)
            for i, (wt, b, act) in enumerate(layers):
                acts[(part, i)] = x
                n, k = wt.shape
                y = torch.empty((B, n), device="cuda")
                la = (B, n, k, x.data_ptr(), x.stride(0), wt.data_ptr(), b.data_ptr(),
                      abi.ACTS[act], y.data_ptr(), n, stream.cuda_stream)
                t_by[(part, i)] = _back_to_back_time(lambda: lib.linear_bias_act(*la), stream,
                                                     20, 3)
                mlp_t += t_by[(part, i)]
                mlp_f += 2.0 * B * n * k
                x = y
        mlp_fwd = None
        if 7137 <= B <= 8192:
            arr = abi._layer_array(bl, "bottom", [])
            yb = torch.empty((B, D), device="cuda")
            ca = (B, len(bl), arr, dense_in.data_ptr(), dense_in.stride(0), yb.data_ptr(), D,
                  stream.cuda_stream)
            t_bottom = _back_to_back_time(lambda: lib.mlp_forward(*ca), stream, 20, 3)
            (w1, b1, a1), (wh, bh, ah) = tl[-2], tl[-1]
            xh = acts[("top", len(tl) - 2)]
            yh = torch.empty((B, 1), device="cuda")
            ha = (B, w1.shape[0], w1.shape[1], xh.data_ptr(), xh.stride(0), w1.data_ptr(),
                  b1.data_ptr(), abi.ACTS[a1], wh.data_ptr(), bh.data_ptr(), abi.ACTS[ah],
                  yh.data_ptr(), 1, stream.cuda_stream)
            t_head = _back_to_back_time(lambda: lib.linear_bias_act_head(*ha), stream, 20, 3)
            mlp_fwd = (t_bottom + sum(t_by[("top", i)] for i in range(len(tl) - 2)) + t_head)
        tf = mlp_f / (mlp_t * 1e-3) / 1e12
        gbs = emb_bytes / (t_emb * 1e-3) / 1e9
        cgbs = emb_comp / (t_emb * 1e-3) / 1e9
        rest = t_fwd - t_emb
        cell = {"batch": B, "forward_us": t_fwd * 1e3, "samples_per_s": B / (t_fwd * 1e-3),
                "emb_interact_us": t_emb * 1e3, "emb_interact_logical_gbps": gbs,
                "emb_interact_compulsory_gbps": cgbs,
                "emb_interact_compulsory_frac": cgbs / HBM_PEAK_GBPS,
                "forward_minus_emb_interact_us": rest * 1e3,
                "forward_minus_emb_interact_tflops": mlp_f / (rest * 1e-3) / 1e12,
                "mlp_layers_us": mlp_t * 1e3, "mlp_layers_tflops": tf,
                "mlp_layers_frac_f32_mfma": tf / F32_MFMA_PEAK_TFLOPS}
        msg = (f"sweep-forward B={B:5d}: forward {t_fwd * 1e3:7.1f} us "
               f"({B / (t_fwd * 1e-3) / 1e6:5.1f} M/s), emb+interact {t_emb * 1e3:6.1f} us "
               f"({gbs:6.0f} GB/s logical, {cgbs:6.0f} compulsory), forward - emb+interact "
               f"{rest * 1e3:6.1f} us, the six layers alone {mlp_t * 1e3:6.1f} us "
               f"({tf:5.1f} TFLOP/s)")
        if mlp_fwd is not None:
            tf_fwd = mlp_f / (mlp_fwd * 1e-3) / 1e12
            cell.update({"mlp_us": mlp_fwd * 1e3, "mlp_tflops": tf_fwd,
                         "mlp_frac_f32_mfma": tf_fwd / F32_MFMA_PEAK_TFLOPS})
            msg += f", the forward's MLP launches alone {mlp_fwd * 1e3:6.1f} us ({tf_fwd:5.1f})"
        cells.append(cell)
        log(msg)
        del ws, out, d64, r
    return {"workload": f"dlrm: {w.description}", "cache": "cold forward and gather, warm "
            "MLP layers (back to back)", "cells": cells}


def copy_rate(stream, mib=1024, reps=10):
    """Read + write rate of a plain 1 GiB device copy (a practical HBM figure)."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        dst.copy_(src)
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize()
    return 2 * (mib << 20) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def host_inclusive_time(case, steps, cold, flush_buf, stream):
    """Median wall time (ms) of one call plus the stream synchronization that
    waits for it: what a caller that needs the result on return sees."""
    import torch
    times = []
    with torch.cuda.stream(stream):
        for s in range(steps):
            if cold:
                flush_buf.max()
            stream.synchronize()
            t0 = time.perf_counter()
            case.run(s)
            stream.synchronize()
            times.append(time.perf_counter() - t0)
    return statistics.median(times) * 1e3


def device_info():
    """The platform figures the rooflines assume, as the runtime reports them."""
    import torch
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "hbm_bytes": p.total_memory, "warp_size": getattr(p, "warp_size", None)}
    for key in ("L2_cache_size", "shared_memory_per_block", "shared_memory_per_multiprocessor",
                "max_threads_per_multi_processor", "regs_per_multiprocessor"):
        if hasattr(p, key):
            info[key] = getattr(p, key)
    return info


def bench_uniform(case, args, stream, flush, cold, practical=None):
    """The benchmark launch with uniform indices (nc32-uniform: the same
    tables, every gathered row a distinct draw, so L2 reuse is negligible and
    the algorithmic bytes are what HBM must deliver)."""
    from dlrm_embedding_bag_amd import inputs
    w = inputs.WORKLOADS["nc32-uniform"]
    ucase = EmbInteractCase(w, args.batches, args.seed, stream, tables=case.tables)
    times, _ = time_steps(ucase, args.steps, args.warmup, cold, flush, stream)
    kms = statistics.mean(time_kernel(ucase, args.steps, args.warmup, cold, flush, stream))
    ms = statistics.mean(times)
    nbytes = ucase.bytes_per_launch()
    dfrac = ucase.distinct_rows_fraction()
    comp = ucase.compulsory_bytes_per_launch(dfrac)
    res = {"workload": f"{w.name}: {w.description}", "us": ms * 1e3, "kernel_us": kms * 1e3,
           "samples_per_s": ucase.B / (ms * 1e-3), "logical_bytes_per_launch": nbytes,
           "distinct_row_fraction": dfrac, "compulsory_bytes_per_launch": comp,
           "kernel_logical_gbps": nbytes / (kms * 1e-3) / 1e9,
           "kernel_compulsory_gbps": comp / (kms * 1e-3) / 1e9,
           "compulsory_frac_of_spec": comp / (kms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    if practical:
        res["compulsory_frac_of_practical_peak"] = (comp / (kms * 1e-3) / 1e9) / practical["gbps"]
    log(f"uniform indices: {ms * 1000:.1f} us per step, kernel {kms * 1000:.1f} us, "
        f"{res['kernel_compulsory_gbps']:.0f} GB/s of distinct bytes "
        f"({res['compulsory_frac_of_spec']:.3f} of 8 TB/s)")
    del ucase
    return res


def profile_linear(shape, stream):
    """Ten launches of one linear layer, 8192 x N x K with A's row stride LDA
    and ReLU, for kernel-trace and counter runs."""
    import torch
    from dlrm_embedding_bag_amd import abi
    N, K, lda = shape
    M = 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(M, lda, device="cuda", generator=g)
    w = torch.randn(N, K, device="cuda", generator=g) * 0.05
    b = torch.randn(N, device="cuda", generator=g)
    c = torch.empty(M, N, device="cuda")
    lib = abi.load()
    for _ in range(10):
        rc = lib.linear_bias_act(M, N, K, a.data_ptr(), lda, w.data_ptr(), b.data_ptr(),
                                 abi.ACTS["relu"], c.data_ptr(), N, stream.cuda_stream)
        if rc:
            raise RuntimeError(f"linear_bias_act: {rc}")
    torch.cuda.synchronize()
    log(f"profile-linear {M}x{N}x{K} (lda {lda}): 10 launches done")


def profile_forward(batches, args, stream):
    """Twelve cold forwards (1 GiB read before each) of the full DLRMv1 model
    at each batch, for kernel-trace and counter runs; prints the median
    event-timed forward of the last eleven."""
    import dataclasses
    import torch
    from dlrm_embedding_bag_amd import abi, inputs
    w = dataclasses.replace(inputs.WORKLOADS["dlrm"], batch=max(batches))
    tables = [inputs.table_device(w, k, args.seed) for k in range(w.num_tables)]
    idx = [torch.from_numpy(inputs.indices(w, k, args.seed)).cuda() for k in range(w.num_tables)]
    dense_in = torch.from_numpy(inputs.dense(w, args.seed)).cuda()
    bottom, top = inputs.dlrm_layers(w, args.seed)
    dev = lambda a: torch.from_numpy(a).cuda()
    model = abi.DlrmModel([(dev(a), dev(b), act) for a, b, act in bottom],
                          [(dev(a), dev(b), act) for a, b, act in top], tables)
    lib = abi.load()
    flush = torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda")
    for B in batches:
        xs = [i[: B * w.bag] for i in idx]
        ws = torch.empty(model.workspace_bytes(B), dtype=torch.uint8, device="cuda")
        out = torch.empty((B, 1), device="cuda")
        fa = (ctypes.byref(model.struct), B, dense_in.data_ptr(), abi._ptr_array(xs), None,
              abi._i64_array([x.numel() for x in xs]), out.data_ptr(), ws.data_ptr(), ws.numel(),
              stream.cuda_stream)
        torch.cuda.synchronize()
        evs = []
        with torch.cuda.stream(stream):
            for _ in range(12):
                if not args.warm:
                    flush.max()
                e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                e[0].record(stream)
                rc = lib.dlrm_forward(*fa)
                if rc:
                    raise RuntimeError(f"dlrm_forward: {rc}")
                e[1].record(stream)
                evs.append(e)
        torch.cuda.synchronize()
        t = statistics.median(a.elapsed_time(b) for a, b in evs[1:])
        log(f"profile-forward B={B}: {t * 1e3:.1f} us per forward "
            f"({'warm' if args.warm else 'cold'}, median of 11)")


def copy_calibration(stream):
    """A plain device copy of 1 GiB, the known-size reference for the HBM
    byte counters (FETCH_SIZE should read 1 GiB, WRITE_SIZE 1 GiB)."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(5):
            dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 5 copies of 1 GiB done")


def _dispatch_counter(run_dir, counter, kernel_part):
    """Median over the dispatches of kernels whose name holds `kernel_part`
    of one counter's per-dispatch total, from a rocprofv3 --pmc output
    directory (its *counter_collection.csv)."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter and kernel_part in row["Kernel_Name"]:
                    key = (fn, row["Dispatch_Id"])
                    per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise ValueError(f"{counter} of a '{kernel_part}' kernel not found under {run_dir}")
    return statistics.median(per.values()), len(per)


DRAM_COUNTERS = ("TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
READ_PROBE_BYTES = 1 << 30


def read_probe(stream, reps=5):
    """Five streaming reads of a 1 GiB buffer (dlrm_stream_read), the
    known-size read that calibrates the FETCH_SIZE counter."""
    import torch
    from dlrm_embedding_bag_amd import abi
    buf = torch.zeros(READ_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(reps):
            abi.dlrm_stream_read(buf, sink, stream=stream)
    torch.cuda.synchronize()
    log(f"read probe: {reps} reads of 1 GiB done")


def record_counters(run_root, workload, kernel_part="interact_kernel"):
    """Memory-side bytes per launch of the workload's kernel from rocprofv3
    --pmc runs, stored in profiles/counters.json under the current kernel
    source hash.  Expects these rocprofv3 -d directories under run_root:

      pmc_<workload>_FETCH_SIZE, pmc_<workload>_WRITE_SIZE   the workload
      pmc_read_FETCH_SIZE    bench.py --read-probe (1 GiB read per dispatch)
      pmc_copy_WRITE_SIZE    bench.py --copy-calibration (1 GiB copy)
      pmc_<workload>_DRAM, pmc_read_DRAM   (optional) TCC_EA0_RDREQ_DRAM_32B_sum
                             and TCC_EA0_WRREQ_WRITE_DRAM_32B_sum, counted in
                             32-byte units, so they need no calibration

    FETCH_SIZE (KiB per dispatch) is scaled by what it reads for the known
    1 GiB streaming read, WRITE_SIZE by what it reads for the 1 GiB copy."""
    d = lambda name: os.path.join(run_root, name)
    fetch, nf = _dispatch_counter(d(f"pmc_{workload}_FETCH_SIZE"), "FETCH_SIZE", kernel_part)
    write, nw = _dispatch_counter(d(f"pmc_{workload}_WRITE_SIZE"), "WRITE_SIZE", kernel_part)
    rfetch, _ = _dispatch_counter(d("pmc_read_FETCH_SIZE"), "FETCH_SIZE", "stream_read_kernel")
    cwrite, _ = _dispatch_counter(d("pmc_copy_WRITE_SIZE"), "WRITE_SIZE", "copyBuffer")
    fscale = READ_PROBE_BYTES / (rfetch * 1024)
    wscale = READ_PROBE_BYTES / (cwrite * 1024)
    entry = {"kernel_source_hash": kernel_source_hash(), "kernel_name_part": kernel_part,
             "dispatches": [nf, nw],
             "fetch_size_kib_per_dispatch": fetch, "write_size_kib_per_dispatch": write,
             "read_probe_fetch_size_kib": rfetch, "copy_write_size_kib": cwrite,
             "calibration_bytes": READ_PROBE_BYTES, "fetch_scale": fscale, "write_scale": wscale,
             "hbm_bytes_per_launch": fetch * 1024 * fscale + write * 1024 * wscale,
             "hbm_read_bytes_per_launch": fetch * 1024 * fscale,
             "hbm_write_bytes_per_launch": write * 1024 * wscale}
    if os.path.isdir(d(f"pmc_{workload}_DRAM")):
        rd, _ = _dispatch_counter(d(f"pmc_{workload}_DRAM"), DRAM_COUNTERS[0], kernel_part)
        wr, _ = _dispatch_counter(d(f"pmc_{workload}_DRAM"), DRAM_COUNTERS[1], kernel_part)
        entry["dram_read_bytes_per_launch"] = rd * 32
        entry["dram_write_bytes_per_launch"] = wr * 32
        entry["dram_bytes_per_launch"] = (rd + wr) * 32
    if os.path.isdir(d("pmc_read_DRAM")):
        prd, _ = _dispatch_counter(d("pmc_read_DRAM"), DRAM_COUNTERS[0], "stream_read_kernel")
        entry["read_probe_dram_read_bytes"] = prd * 32
    try:
        with open(COUNTERS_JSON) as f:
            allc = json.load(f)
    except (OSError, ValueError):
        allc = {}
    allc[workload] = entry
    with open(COUNTERS_JSON, "w") as f:
        json.dump(allc, f, indent=1)
        f.write("\n")
    return entry


def forward_penalty(args, stream):
    """Where the B=8192 forward's MLP launches lose time against their
    standalone runs: the cold forward with and without every MLP weight
    read back into the caches after the flush, the top launches back to
    back alone, in pairs, and after the gather, and top layer 0 alone on a
    warm and a cold A."""
    import torch
    from dlrm_embedding_bag_amd import abi, inputs
    w = inputs.WORKLOADS["dlrm"]
    B = w.batch
    tables = [inputs.table_device(w, k, args.seed) for k in range(w.num_tables)]
    idx = [torch.from_numpy(inputs.indices(w, k, args.seed)).cuda() for k in range(w.num_tables)]
    dense_in = torch.from_numpy(inputs.dense(w, args.seed)).cuda()
    bottom, top = inputs.dlrm_layers(w, args.seed)
    dev = lambda a: torch.from_numpy(a).cuda()
    bl = [(dev(a), dev(b), act) for a, b, act in bottom]
    tl = [(dev(a), dev(b), act) for a, b, act in top]
    model = abi.DlrmModel(bl, tl, tables)
    flush = torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda")
    out = abi.dlrm_forward(model, dense_in, idx, stream=stream)
    sink = torch.zeros(1, device="cuda")
    weights = [x[0] for x in bl + tl]
    for warm in (False, True):
        ts = []
        for it in range(25):
            with torch.cuda.stream(stream):
                flush.max()
                if warm:
                    for t in weights:
                        sink += t.sum()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                abi.dlrm_forward(model, dense_in, idx, out=out, stream=stream)
                e1.record(stream)
            torch.cuda.synchronize()
            if it >= 5:
                ts.append(e0.elapsed_time(e1) * 1000)
        log(f"forward-penalty: forward {'with the MLP weights read after the flush' if warm else 'cold'}"
            f": {statistics.median(ts):.1f} us")
    lib = abi.load()
    d = abi.mlp_forward(dense_in, bl, stream=stream)
    R = abi.dlrm_emb_interact(tables, idx, d, stream=stream)
    H = torch.empty(B, tl[0][0].shape[0], device="cuda")
    o = torch.empty(B, 1, device="cuda")
    (w0, b0, a0), (w1, b1, a1), (w2, b2, a2) = tl
    t0 = (B, w0.shape[0], w0.shape[1], R.data_ptr(), R.stride(0), w0.data_ptr(), b0.data_ptr(),
          abi.ACTS[a0], H.data_ptr(), H.stride(0), stream.cuda_stream)
    t1 = (B, w1.shape[0], w1.shape[1], H.data_ptr(), H.stride(0), w1.data_ptr(), b1.data_ptr(),
          abi.ACTS[a1], w2.data_ptr(), b2.data_ptr(), abi.ACTS[a2], o.data_ptr(), 1,
          stream.cuda_stream)
    top0 = lambda: lib.linear_bias_act(*t0)
    top1 = lambda: lib.linear_bias_act_head(*t1)
    gather = lambda: abi.dlrm_emb_interact(tables, idx, d, out=R, stream=stream)
    torch.cuda.synchronize()
    a = _back_to_back_time(top0, stream)
    b = _back_to_back_time(top1, stream)
    p = _back_to_back_time(lambda: (top0(), top1()), stream)
    g = _back_to_back_time(gather, stream, launches=10)
    q = _back_to_back_time(lambda: (gather(), top0(), top1()), stream, launches=10)
    log(f"forward-penalty: back to back, per launch or sequence: top 0 {a * 1e3:.1f} us, "
        f"top 1 + head {b * 1e3:.1f}, the two alternating {p * 1e3:.1f}, gather + interaction "
        f"{g * 1e3:.1f}, gather then both {q * 1e3:.1f}")
    # Top 0 alone on a warm and on a cold A (the cache flush before each
    # launch), with R's rows 415 floats apart (dword-aligned loads) and
    # padded to 416 as inside the forward (16-byte loads).
    Rp = torch.zeros((B, R.shape[1] + 1), device="cuda")
    Rp[:, :R.shape[1]] = R
    for name, A, lda in (("stride 416", Rp, Rp.stride(0)), ("stride 415", R, R.stride(0))):
        ta = (B, w0.shape[0], w0.shape[1], A.data_ptr(), lda, w0.data_ptr(), b0.data_ptr(),
              abi.ACTS[a0], H.data_ptr(), H.stride(0), stream.cuda_stream)
        warm = _back_to_back_time(lambda: lib.linear_bias_act(*ta), stream, launches=20)
        ts = []
        for it in range(25):
            with torch.cuda.stream(stream):
                flush.max()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                lib.linear_bias_act(*ta)
                e1.record(stream)
            torch.cuda.synchronize()
            if it >= 5:
                ts.append(e0.elapsed_time(e1) * 1000)
        log(f"forward-penalty: top 0 alone, A {name}: warm {warm * 1e3:.1f} us, cold "
            f"{statistics.median(ts):.1f} us")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="nc32")
    ap.add_argument("--batches", type=int, default=4, help="distinct index batches to rotate")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--warm", action="store_true", help="do not flush caches between steps")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only five 1 GiB device copies (the WRITE_SIZE calibration)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only five 1 GiB streaming reads (the FETCH_SIZE calibration)")
    ap.add_argument("--record-counters", metavar="DIR", default="",
                    help="store the workload's HBM bytes per launch from rocprofv3 --pmc "
                         "runs under DIR in profiles/counters.json (no GPU needed)")
    ap.add_argument("--no-forward", action="store_true",
                    help="skip the full-forward section (B=8192 DLRMv1)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the bf16 / mean / weighted / CSR variant lines")
    ap.add_argument("--no-cells", action="store_true",
                    help="skip the pages' small-cell forward latency grid (eager vs plan)")
    ap.add_argument("--sweep", action="store_true", help="batch x num_tables sweep instead")
    ap.add_argument("--sweep-forward", action="store_true",
                    help="batch sweep of the full forward instead")
    ap.add_argument("--sweep-steps", type=int, default=10)
    ap.add_argument("--sweep-out", default="")
    ap.add_argument("--profile-linear", type=int, nargs=3, metavar=("N", "K", "LDA"),
                    help="only 10 launches of one 8192-row linear layer (for counter runs)")
    ap.add_argument("--profile-run", action="store_true",
                    help="only the cold timed steps (for profiler runs)")
    ap.add_argument("--forward-penalty", action="store_true",
                    help="the B=8192 forward's MLP launches in and out of the forward")
    ap.add_argument("--profile-forward", default="", metavar="B1,B2,...",
                    help="only twelve cold forwards of the full DLRMv1 model at each batch "
                         "(for profiler runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.record_counters:
        print(json.dumps(record_counters(args.record_counters, args.workload), indent=1))
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    from dlrm_embedding_bag_amd import abi
    if not os.path.exists(abi.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    stream = torch.cuda.Stream()
    if args.copy_calibration:
        copy_calibration(stream)
        return
    if args.read_probe:
        read_probe(stream)
        return
    if args.profile_linear:
        profile_linear(args.profile_linear, stream)
        return
    if args.profile_forward:
        profile_forward([int(b) for b in args.profile_forward.split(",")], args, stream)
        return
    if args.forward_penalty:
        forward_penalty(args, stream)
        return
    if args.sweep_forward:
        import torch
        flush = torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda")
        res = bench_sweep_forward(args, stream, flush)
        if args.sweep_out:
            with open(args.sweep_out, "w") as f:
                json.dump(res, f, indent=1)
        print(json.dumps(res), flush=True)
        return
    if args.sweep:
        import torch
        flush = torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda")
        res = bench_sweep(args, stream, flush)
        if args.sweep_out:
            with open(args.sweep_out, "w") as f:
                json.dump(res, f, indent=1)
        print(json.dumps(res), flush=True)
        return
    if args.workload in VARIANTS:
        res = bench_variant_line(args, stream)
        print(json.dumps(res), flush=True)
        return
    res = bench_emb_interact(args, stream)
    if not args.profile_run:
        import torch
        flush = torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda")
        if not args.no_variants:
            res["variants"] = bench_variants(args, stream, flush)
        if not args.no_cells:
            res["cells"] = bench_cells(args, stream)
        if not args.no_forward:
            res["forward"] = bench_forward(args, stream, flush)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
