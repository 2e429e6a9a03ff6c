"""Decode-attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama3_8b_gqa]

One step is one pass of the whole hot path over one batch: the fused NeoX
RoPE + paged-KV append of the new token (lgm_rope_kv_append), then split-K
paged GQA decode attention with its log-sum-exp merge (lgm_paged_decode_attn),
all through the C ABI on torch's current stream, inputs resident in HBM.

Printed: one JSON line with the KV bandwidth of the whole step (value, GB/s),
tokens/s, the roofline of the attention launch (algorithmic KV bytes per
launch over its average duration, timed with HIP events on its stream) and
the fp64 CPU oracle timed on the host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention KV GB/s (% of HBM peak) + tokens/s, 1 MI355X"
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "paged_gqa_decode_lgm_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kv_bytes: int):
    """HBM bytes per attention launch from committed rocprofv3 PMC runs, if they
    were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def _oracle_passes(w, threads: int, min_seconds: float, max_passes: int):
    """Times the fp64 oracle over the whole batch under a BLAS/OpenMP thread
    limit; passes repeat until ~min_seconds of work.  Returns the pass times."""
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import append as OAP
    from oracle import attention as OA

    c = w.cfg
    kp, vp = W.storage_bits(w.k_pool), W.storage_bits(w.v_pool)
    q = OAP.act_to_f64(W.storage_bits(w.qkv)[:, : c.num_q_heads * c.head_dim], c.act).reshape(
        c.num_seqs, c.num_q_heads, c.head_dim)
    times = []
    with threadpool_limits(threads):
        while len(times) < max_passes and (not times or sum(times) < min_seconds):
            t0 = time.perf_counter()
            OA.paged_decode(q, kp, vp, w.block_tables.numpy(), w.context_lens.numpy(), c.softmax_scale,
                            num_kv_heads=c.num_kv_heads, block_size=c.block_size, cache=c.cache,
                            k_scale=None if w.k_scale is None else w.k_scale.numpy(),
                            v_scale=None if w.v_scale is None else w.v_scale.numpy())
            times.append(time.perf_counter() - t0)
    return times


def host_threads() -> int:
    """Cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS when that is set."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(n, 1)


def cpu_baseline(w, min_seconds: float = 12.0, max_passes: int = 10):
    """The fp64 oracle on the whole batch (host copies of the same inputs),
    one thread; the median pass is kept.  The same run with the BLAS/OpenMP
    pools at every available core is reported beside it."""
    c = w.cfg
    times = _oracle_passes(w, 1, min_seconds, max_passes)
    t = statistics.median(times)
    n = host_threads()
    times_n = _oracle_passes(w, n, min_seconds / 2, max_passes)
    tn = statistics.median(times_n)
    return {"value": round(w.kv_bytes() / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tokens_per_s": round(c.num_seqs / t, 3),
            "sample": f"attention over the whole {c.name} batch ({c.num_seqs} sequences, "
                      f"{int(w.context_lens.sum())} cached tokens) in fp64 NumPy, 1 thread, median of "
                      f"{len(times)} passes of {t:.2f} s",
            "all_cores": {"value": round(w.kv_bytes() / tn / 1e9, 4), "unit": "GB/s", "cores": n,
                          "tokens_per_s": round(c.num_seqs / tn, 3),
                          "sample": f"the same, BLAS/OpenMP pools limited to {n} threads, median of "
                                    f"{len(times_n)} passes of {tn:.2f} s"}}


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence.

    Recording a default event (as torch's are) ends in a system-scope cache
    write-back and invalidate; between back-to-back calls that costs the GPU
    a couple of microseconds per record and slows the launch that follows.
    Timing needs no such fence: the host reads the events only after a
    device synchronisation.  Interface: record(stream), synchronize(),
    elapsed_time(end) in milliseconds."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence, hip_runtime_api.h
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes

            import torch

            torch.cuda.init()
            # The HIP runtime torch already loaded: events must belong to it.
            path = None
            with open("/proc/self/maps") as fh:
                for line in fh:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("TimingEvent: the HIP runtime is not loaded")
            lib = ctypes.CDLL(path)
            vp, u = ctypes.c_void_p, ctypes.c_uint
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), u]
            lib.hipEventRecord.argtypes = [vp, vp]
            lib.hipEventSynchronize.argtypes = [vp]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            lib.hipEventDestroy.argtypes = [vp]
            lib.hipGetErrorString.argtypes = [ctypes.c_int]
            lib.hipGetErrorString.restype = ctypes.c_char_p
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes

        self._ctypes = ctypes
        lib = self._lib()
        self._h = ctypes.c_void_p()
        self._check(lib.hipEventCreateWithFlags(ctypes.byref(self._h), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")

    def _check(self, rc: int, what: str) -> None:
        if rc != 0:
            raise RuntimeError(f"{what}: {self._hip.hipGetErrorString(rc).decode()} ({rc})")

    def record(self, stream) -> None:
        self._check(self._hip.hipEventRecord(self._h, self._ctypes.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def synchronize(self) -> None:
        self._check(self._hip.hipEventSynchronize(self._h), "hipEventSynchronize")

    def elapsed_time(self, end: "TimingEvent") -> float:
        end.synchronize()
        ms = self._ctypes.c_float()
        self._check(self._hip.hipEventElapsedTime(self._ctypes.byref(ms), self._h, end._h), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        try:
            if self._h:
                self._hip.hipEventDestroy(self._h)
        except Exception:
            pass


def read_ceiling(torch, nbytes: int = 4 << 30, reps: int = 10):
    """The measured streaming ceiling: lgm_stream_read_probe over an nbytes
    buffer, for a few workgroup counts with and without the non-temporal
    hint; the fastest median is the ceiling."""
    from paged_gqa_decode_lgm_amd import _binding as Bn

    dev = torch.device("cuda:0")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    best = None
    for nwg in (1024, 2048, 4096):
        for nt in (1, 0):
            call = lambda: Bn.lgm_stream_read_probe(buf, nbytes, nwg, nt, sink)
            call()
            ms = []
            for _ in range(reps):
                a, b = TimingEvent(), TimingEvent()
                a.record(stream)
                call()
                b.record(stream)
                b.synchronize()
                ms.append(a.elapsed_time(b))
            gbs = nbytes / (statistics.median(ms) / 1e3) / 1e9
            if best is None or gbs > best["gbs"]:
                best = {"gbs": round(gbs, 1), "workgroups": nwg, "nontemporal": bool(nt)}
    del buf
    best.update({"probe": f"read-only stream of {nbytes >> 30} GiB, 16-byte loads, median of {reps}",
                 "pct_of_hbm_peak": round(100.0 * best["gbs"] / HBM_PEAK_GBS, 2)})
    return best


def _quantile(xs, q: float) -> float:
    ys = sorted(xs)
    return ys[min(len(ys) - 1, int(q * len(ys)))]


ATTN_KERNELS = ("paged_decode", "merge")  # the launches of one lgm_paged_decode_attn call


def copy_probe(nbytes: int, reps: int) -> int:
    """A plain device copy of nbytes, reps times: the known-size kernel that
    scales rocprofv3's FETCH_SIZE / WRITE_SIZE readings to bytes."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)
    return 0


def _counter_means(path: str, counter: str):
    """Mean counter value (KiB) per dispatch for each kernel name in a rocprofv3 counter_collection.csv."""
    import csv
    import collections

    acc = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic_summary(workload: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str,
                    copy_bytes: int, commands: list) -> int:
    """HBM bytes per attention call from two rocprofv3 --pmc runs of the bench (FETCH_SIZE, WRITE_SIZE),
    each scaled by the same counter's reading for the copy probe; writes profiles/traffic_<workload>.json."""
    cf = max(_counter_means(copy_fetch_csv, "FETCH_SIZE").items(), key=lambda kv: kv[1])
    cw = max(_counter_means(copy_write_csv, "WRITE_SIZE").items(), key=lambda kv: kv[1])
    f_fetch = copy_bytes / (cf[1] * 1024.0)
    f_write = copy_bytes / (cw[1] * 1024.0)
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    kernels = {}
    for name in fetch:
        if any(k in name for k in ATTN_KERNELS + ("paged_mla",)):
            kernels[name] = {"fetch_bytes": fetch[name] * 1024.0 * f_fetch,
                             "write_bytes": write.get(name, 0.0) * 1024.0 * f_write}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in kernels.values())
    rec = {"workload": workload, "kernel_source_hash": kernel_source_hash(), "hbm_bytes_per_launch": total,
           "copy_probe": {"bytes": copy_bytes, "kernel": cf[0], "fetch_kib": cf[1], "write_kib": cw[1],
                          "fetch_scale": f_fetch, "write_scale": f_write},
           "kernels": kernels, "commands": commands}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))
    return 0


# MI355X: 256 compute units of 4 SIMDs in 8 XCDs (GRBM_GUI_ACTIVE is counted once per XCD).
NUM_CU, SIMD_PER_CU, NUM_XCD = 256, 4, 8


def _dispatch_counters(paths):
    """{kernel: {counter: [value per dispatch]}} from rocprofv3 counter_collection.csv files; the rows of
    one dispatch and counter (one per hardware instance, or one already summed) are added."""
    import csv
    import collections

    per = collections.defaultdict(float)
    names = {}
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                key = (path, r["Dispatch_Id"], r["Counter_Name"])
                per[key] += float(r["Counter_Value"])
                names[(path, r["Dispatch_Id"])] = r["Kernel_Name"]
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for (path, disp, counter), v in per.items():
        out[names[(path, disp)]][counter].append(v)
    return out


def counter_summary(workload: str, paths, commands: list) -> int:
    """Per-kernel means of the SQ/GRBM counters of rocprofv3 --pmc runs of the bench, and the shares they
    give (wave-lifetime shares of VALU issue, memory issue and waiting; MFMA busy per SIMD-cycle of the
    kernel's span); writes profiles/counters_<workload>.json."""
    data = _dispatch_counters(paths)
    kernels = {}
    for name, cs in data.items():
        if not any(k in name for k in ATTN_KERNELS + ("paged_mla", "rope_kv_append")):
            continue
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        rec = {"dispatches": max(len(v) for v in cs.values()), "counters": mean}
        wave = mean.get("SQ_WAVE_CYCLES")
        gui = mean.get("GRBM_GUI_ACTIVE")
        derived = {}
        if wave:
            for c, label in (("SQ_ACTIVE_INST_VALU", "valu_active_share_of_wave_cycles"),
                             ("SQ_ACTIVE_INST_VMEM", "vmem_issue_share_of_wave_cycles"),
                             ("SQ_WAIT_INST_ANY", "wait_inst_any_share_of_wave_cycles"),
                             ("SQ_WAIT_ANY", "wait_any_share_of_wave_cycles"),
                             ("SQ_ACTIVE_INST_ANY", "any_issue_share_of_wave_cycles")):
                if c in mean:
                    derived[label] = round(mean[c] / wave, 4)
        if gui:
            span = gui / NUM_XCD  # cycles of the kernel's span, per XCD
            derived["span_cycles_per_xcd"] = round(span, 1)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                derived["mfma_busy_pct"] = round(100.0 * mean["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                                 (span * NUM_CU * SIMD_PER_CU), 2)
            if "SQ_ACTIVE_INST_VALU" in mean:
                derived["valu_busy_pct"] = round(100.0 * mean["SQ_ACTIVE_INST_VALU"] / NUM_CU / span, 2)
            if "SQ_BUSY_CYCLES" in mean:
                derived["sq_busy_cycles_per_xcd"] = round(mean["SQ_BUSY_CYCLES"] / NUM_XCD, 1)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in mean:  # 512 flops per MOP (rocprofv3's own derived metrics)
            derived["mfma_bf16_flops_per_dispatch"] = round(512.0 * mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"], 1)
        if mean.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in mean:
            derived["valu_coexec_share_of_mfma_busy"] = round(mean["SQ_VALU_MFMA_COEXEC_CYCLES"] /
                                                              mean["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
        if "SQ_WAVES" in mean and mean["SQ_WAVES"]:
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_BF16", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU",
                      "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS"):
                if c in mean:
                    derived[c.lower().replace("sq_insts_", "insts_per_wave_")] = round(mean[c] / mean["SQ_WAVES"], 1)
        rec["derived"] = derived
        kernels[name] = rec
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(), "kernels": kernels,
           "commands": commands,
           "notes": "counters summed over hardware instances per dispatch, then averaged over dispatches; "
                    "SQ_WAVE_CYCLES, SQ_ACTIVE_INST_*, SQ_WAIT_* in the same (quad-cycle) units; "
                    f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {NUM_XCD} * {NUM_CU * SIMD_PER_CU} "
                    f"SIMDs); VALU busy = SQ_ACTIVE_INST_VALU / {NUM_CU} CUs / (GRBM_GUI_ACTIVE / {NUM_XCD})"}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"counters_{workload}.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    return 0


MLA_METRIC = "MLA latent decode KV GB/s (% of HBM peak) + us/token, 1 MI355X"


def mla_cpu_baseline(w, min_seconds: float = 10.0, max_passes: int = 50):
    """The fp64 MLA oracle on the whole batch, one thread (median pass)."""
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import codecs
    from oracle import mla as OM

    c = w.cfg
    q_lat = codecs.bf16_decode(W.storage_bits(w.q_latent))
    q_pe = codecs.bf16_decode(W.storage_bits(w.q_pe))
    ckv, kpe = W.storage_bits(w.ckv_pool), W.storage_bits(w.kpe_pool)
    scale = float(w.ckv_scale[0]) if w.ckv_scale is not None else 1.0
    times = []
    with threadpool_limits(1):
        while len(times) < max_passes and (not times or sum(times) < min_seconds):
            t0 = time.perf_counter()
            OM.paged_mla_decode(q_lat, q_pe, ckv, kpe, w.block_tables.numpy(), w.context_lens.numpy(),
                                c.softmax_scale, block_size=c.block_size, ckv_cache=c.ckv_cache, ckv_scale=scale)
            times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": round(w.kv_bytes() / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "us_per_token": round(t * 1e6 / c.num_seqs, 1),
            "sample": f"MLA decode over the whole {c.name} batch ({c.num_seqs} sequences, "
                      f"{int(w.context_lens.sum())} cached tokens) in fp64 NumPy, 1 thread, median of "
                      f"{len(times)} passes of {t:.3f} s"}


def run_mla(args, torch, W) -> int:
    """One step = one lgm_paged_mla_decode call (split-K latent decode and its
    LSE merge: two launches) over the workload's batch.  The call is captured
    once in a HIP graph and the graph replayed back to back (the eager call's
    host overhead exceeds its GPU time at one sequence); every replay's output
    is compared bitwise with the eager call's."""
    from paged_gqa_decode_lgm_amd import ops

    cfg = W.MLA_CONFIGS[args.workload]
    if args.partition_size is not None:
        cfg = cfg.with_(partition_size=args.partition_size)
    w = W.make_mla_workload(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cu = lambda t: None if t is None else t.to(dev)
    ql, qp, ckv, kpe = cu(w.q_latent), cu(w.q_pe), cu(w.ckv_pool), cu(w.kpe_pool)
    bt, ctx, sc = cu(w.block_tables), cu(w.context_lens), cu(w.ckv_scale)
    B, H = cfg.num_seqs, cfg.num_heads
    max_ctx = int(w.context_lens.max())
    ps_arg = cfg.partition_size if args.partition_size is not None else 0
    ps = ops.mla_partition_size(ql, qp, ckv, bt, max_ctx, ps_arg)
    ws_bytes = ops.mla_workspace_bytes(ql, qp, ckv, bt, max_ctx, ps_arg)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, cfg.latent_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    call = lambda: ops.paged_mla_decode(ql, qp, ckv, kpe, bt, ctx, max_ctx, cfg.softmax_scale, sc,
                                        partition_size=ps_arg, out=out, out_lse=lse, workspace=ws)
    call()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(args.warmup):
        graph.replay()
    stream = torch.cuda.current_stream()
    events = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
    mismatches = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in events:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for _ in range(3):  # replays interleaved with eager host work, each checked
        graph.replay()
        torch.cuda.synchronize()
        mismatches += int(not (torch.equal(out.view(torch.int16), ref_out.view(torch.int16)) and
                               torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))))
    call_ms = [a.elapsed_time(b) for a, b in events]

    # Eight consecutive calls in one graph, as a model's graph holds one call
    # per layer: one graph launch per eight calls, so that at one sequence the
    # host's launch of the next replay no longer shows in the per-call time.
    n_in = 8
    graph8 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph8):
        for _ in range(n_in):
            call()
    for _ in range(2):
        graph8.replay()
    ev8 = [(TimingEvent(), TimingEvent()) for _ in range(max(args.steps // n_in, 5))]
    torch.cuda.synchronize()
    for a, b in ev8:
        a.record(stream)
        graph8.replay()
        b.record(stream)
    torch.cuda.synchronize()
    per_call8 = [a.elapsed_time(b) / n_in for a, b in ev8]
    out.zero_()
    lse.zero_()
    graph8.replay()
    torch.cuda.synchronize()
    mismatches += int(not (torch.equal(out.view(torch.int16), ref_out.view(torch.int16)) and
                           torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))))

    ms_per_step = wall * 1e3 / args.steps
    kv = w.kv_bytes()
    call_avg_s = statistics.mean(call_ms) / 1e3
    achieved = kv / call_avg_s / 1e9
    value = kv / (ms_per_step / 1e3) / 1e9
    rec = {
        "metric": MLA_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 latent + bf16 rope kv / bf16 act",
        "data": "synthetic (seeded N(0,1) latent and positional rows, FP8 ckv with a calibrated per-tensor scale, "
                "block tables)",
        "config": {"workload": cfg.name, "global_batch": B, "context": cfg.ctx if isinstance(cfg.ctx, int) else
                   list(cfg.ctx), "sum_context_tokens": int(w.context_lens.sum()), "num_heads": H,
                   "latent_dim": cfg.latent_dim, "rope_dim": cfg.rope_dim, "block_size": cfg.block_size,
                   "partition_size": ps, "parallelism": "single GPU"},
        "us_per_token": round(call_avg_s * 1e6 / B, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kv_bytes_per_step": kv,
        "graph_replays_bitwise_equal_to_eager": mismatches == 0,
        "kernel_ms": {"call_avg": round(call_avg_s * 1e3, 5), "call_median": round(statistics.median(call_ms), 5),
                      "call_p10": round(_quantile(call_ms, 0.1), 5), "call_p90": round(_quantile(call_ms, 0.9), 5),
                      "graph_of_8_calls": {"call_avg": round(statistics.mean(per_call8), 5),
                                           "call_median": round(statistics.median(per_call8), 5),
                                           "replays": len(ev8)}},
        "roofline": {"bound": "hbm", "kernel": f"lgm_paged_mla_decode (latent decode in {ps}-token partitions + "
                     "LSE merge, one call: two launches, replayed from a HIP graph)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(cfg.name, kv)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = mla_cpu_baseline(w)
    print(json.dumps(rec), flush=True)
    return 0 if mismatches == 0 else 1


def graph_replay(torch, step, stream, steps: int, outputs) -> dict:
    """The step captured once in a HIP graph and replayed back to back, with
    events around each replay: the GPU time of a step without the host's
    launch overhead (what bounds latency-bound shapes when run eagerly).
    Checked replays, with host synchronisations between them, must equal the
    eager step's outputs bitwise."""
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(5):
        graph.replay()
    events = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in events:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in events]
    equal = True
    for _ in range(3):
        for t in outputs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        equal &= all(torch.equal(t.view(torch.uint8), r.view(torch.uint8)) for t, r in zip(outputs, ref))
    return {"step_avg_ms": round(statistics.mean(ms), 5), "step_median_ms": round(statistics.median(ms), 5),
            "step_p10_ms": round(_quantile(ms, 0.1), 5), "replays": steps,
            "replays_bitwise_equal_to_eager": bool(equal)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b_gqa")
    ap.add_argument("--partition-size", type=int, default=None, help="override the workload's partition size")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a HIP graph (reported under 'graph')")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-only streaming ceiling probe")
    ap.add_argument("--cold", type=int, default=10, help="extra attention calls timed after a cache-evicting write")
    ap.add_argument("--copy-probe", type=int, default=None, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=5, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "COPY_BYTES"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 counter_collection.csv files")
    ap.add_argument("--counter-summary", nargs="+", default=None, metavar="CSV",
                    help="write profiles/counters_<workload>.json from rocprofv3 counter_collection.csv files")
    ap.add_argument("--commands", nargs="*", default=[], help="the profiling command lines, recorded with the summary")
    args = ap.parse_args()
    if args.counter_summary:
        return counter_summary(args.workload, args.counter_summary, args.commands)
    if args.traffic_summary:
        f, w_, cf, cw, cb = args.traffic_summary
        return traffic_summary(args.workload, f, w_, cf, cw, int(cb), args.commands)
    if args.copy_probe:
        return copy_probe(args.copy_probe, max(args.steps, 1))
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the library has no "
              "multi-GPU path (the decode step would shard by kv heads, or by sequence blocks with one "
              "exchange of LSE records before lgm_lse_merge).", file=sys.stderr)
        return 2

    import torch

    import workloads as W
    from paged_gqa_decode_lgm_amd import ops

    if args.workload in W.MLA_CONFIGS:
        return run_mla(args, torch, W)
    cfg = W.CONFIGS[args.workload]
    if args.partition_size is not None:
        cfg = cfg.with_(partition_size=args.partition_size)
    w = W.make_workload(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cu = lambda t: None if t is None else t.to(dev)
    qkv, k_pool, v_pool = cu(w.qkv), cu(w.k_pool), cu(w.v_pool)
    if cfg.cache == W.DTYPE_FP4:
        k_pool = ops.FP4Pool(k_pool, cfg.block_size, cfg.num_kv_heads, cfg.head_dim)
        v_pool = ops.FP4Pool(v_pool, cfg.block_size, cfg.num_kv_heads, cfg.head_dim)
    bt, ctx, ks, vs = cu(w.block_tables), cu(w.context_lens), cu(w.k_scale), cu(w.v_scale)
    max_ctx = int(w.context_lens.max())
    B, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
    q = torch.empty((B, Hq, D), dtype=qkv.dtype, device=dev)
    if not cfg.append:
        q.copy_(qkv[:, : Hq * D].reshape(B, Hq, D))
    out = torch.empty((B, Hq, D), dtype=qkv.dtype, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws_bytes = ops.workspace_bytes(q, k_pool, bt, max_ctx, cfg.partition_size)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)  # zero-filled once, kept zero by the library
    ps = ops.partition_size(q, k_pool, bt, max_ctx, cfg.partition_size)
    stream = torch.cuda.current_stream()

    # Two events per step, around the attention call.  The append of step i
    # runs between the end of step i-1's call and the start of step i's, so
    # that interval times it (with the launch gaps around it) without a third
    # event per step.
    def step(ev=None):
        if cfg.append:
            ops.rope_kv_append(qkv, k_pool, v_pool, bt, ctx, cfg.rope_theta, Hq, ks, vs, q_out=q)
        if ev:
            ev[0].record(stream)
        ops.paged_decode_attn(q, k_pool, v_pool, bt, ctx, max_ctx, softmax_scale=cfg.softmax_scale,
                              partition_size=cfg.partition_size, k_scale=ks, v_scale=vs, out=out, out_lse=lse,
                              workspace=ws)
        if ev:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    events = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    graph_rec = graph_replay(torch, step, stream, args.steps, (q, out, lse)) if args.graph else None

    # Cold calls: reading 1 GiB between calls (outside the event pair) evicts
    # the previous call's lines from L2 and the 256 MB Infinity Cache.  A read,
    # not a write: evicting a write's dirty lines would charge the next call
    # with someone else's write-back traffic.
    scratch = torch.zeros(1 << 27, dtype=torch.int64, device=dev)
    torch.sum(scratch)
    cold_ms = []
    for _ in range(args.cold):
        torch.sum(scratch)
        a, b = TimingEvent(), TimingEvent()
        a.record(stream)
        ops.paged_decode_attn(q, k_pool, v_pool, bt, ctx, max_ctx, softmax_scale=cfg.softmax_scale,
                              partition_size=cfg.partition_size, k_scale=ks, v_scale=vs, out=out, out_lse=lse,
                              workspace=ws)
        b.record(stream)
        b.synchronize()
        cold_ms.append(a.elapsed_time(b))
    del scratch

    attn_ms = [e[0].elapsed_time(e[1]) for e in events]
    # (step 0's append follows an idle GPU and its launch latency: left out)
    append_ms = [events[i - 1][1].elapsed_time(events[i][0]) for i in range(1, len(events))] if cfg.append else []
    ms_per_step = wall * 1e3 / args.steps
    kv = w.kv_bytes()
    attn_avg_s = statistics.mean(attn_ms) / 1e3
    achieved = kv / attn_avg_s / 1e9
    value = kv / (ms_per_step / 1e3) / 1e9
    traffic = measured_traffic(cfg.name, kv)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8-e4m3 kv / bf16 act", "fp4": "fp4-e2m1 (e8m0 per 32) kv / bf16 act"}.get(
            cfg.cache, cfg.cache),
        "data": ("synthetic (seeded uniform E2M1 code bytes and E8M0 scale bytes, N(0,1) packed QKV, block tables)"
                 if cfg.cache == W.DTYPE_FP4 else "synthetic (seeded N(0,1) KV cache, packed QKV and block tables)"),
        "config": {"workload": cfg.name, "global_batch": B, "context": (list(cfg.ctx) if not isinstance(cfg.ctx, int)
                   else cfg.ctx), "sum_context_tokens": int(w.context_lens.sum()), "num_q_heads": Hq,
                   "num_kv_heads": cfg.num_kv_heads, "head_dim": D, "block_size": cfg.block_size,
                   "partition_size": ps, "append": cfg.append, "parallelism": "single GPU"},
        "tokens_per_s": round(B / (ms_per_step / 1e3), 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kv_bytes_per_step": kv,
        "kernel_ms": {"attention_avg": round(attn_avg_s * 1e3, 5),
                      "attention_median": round(statistics.median(attn_ms), 5),
                      "attention_p10": round(_quantile(attn_ms, 0.1), 5),
                      "attention_p90": round(_quantile(attn_ms, 0.9), 5),
                      "append_avg": round(statistics.mean(append_ms), 5) if append_ms else None,
                      "attention_cold_avg": round(statistics.mean(cold_ms), 5) if cold_ms else None},
        "roofline": {"bound": "hbm", "kernel": "lgm_paged_decode_attn (" + (
                     "whole-row decode over equal tile ranges + LSE merge" if ps == 0 else
                     f"split-K decode in {ps}-token partitions + LSE merge; whole-row kernel over equal runs of "
                     "whole partitions when contexts are long, else the work-queue kernel") +
                     ", one call: two launches)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    if graph_rec is not None:
        rec["graph"] = graph_rec
    if not args.no_ceiling:
        ceil = read_ceiling(torch)
        ceil["attention_pct_of_ceiling"] = round(100.0 * achieved / ceil["gbs"], 2)
        rec["ceiling"] = ceil
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
