#!/usr/bin/env python3
"""Benchmark of MLA chunked prefill on one MI355X.

Headline workload (default): the fp8 ragged batch, the largest single-GPU
configuration: one layer, 128 heads, 16 requests with context lengths uniform
in [1024, 32768] (multiples of 64) and 256..2048 new tokens each, c_kv stored
as fp8-e4m3 with one fp32 scale per token beside bf16 k_rope, 64-token blocks
in a shuffled pool, context chunk 4096. A step is one pass of the whole path:
per context chunk gather (fp8 dequantisation) -> kv_b_proj decompression ->
attention -> LSE merge into the running state; the last chunk's attention
also covers the new tokens' keys (decompressed beside the chunk's, causal)
and writes the result. Inputs are seeded synthetic data resident in HBM
before timing starts.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]

Prints one JSON line: TFLOP/s of algorithmic work (2*512*256 flop per
decompressed (token, head), 640 flop per visible (row, key, head)) over the
timed steps (eager launches; --graph replays one step captured into a HIP
graph), prefill tokens/s, the roofline of the dominant kernel (per-launch
duration from HIP events on the launch stream, taken in a second pass of the
same number of steps, since events between launches add fences to the step),
the fp64 CPU oracle timed on a bounded sample on this host's cores, and one
sub-record per other standard workload (bf16 DeepSeek-V3 geometry, long
context, head-partitioned reuse), each with its own dominant kernel's
roofline (--no-sub skips them).

    python bench.py --workload {1..5}   # one standard workload alone
    python bench.py --append            # the cache write path
    python bench.py --artifact          # the offline Local-head artifact build
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MLA chunked-prefill TFLOP/s + prefill tokens/s; % of MFMA/HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
HEADLINE = 4                   # the fp8 ragged batch: the largest single-GPU workload
SUB_WORKLOADS = (2, 3, 5)
CSRC = os.path.join(ROOT, "mla_long_context_amd", "csrc")
# timer span -> (kernel name in rocprofv3 traces, source file) for the HBM
# counter records (the chunked workloads' default schedule: every context
# pass is mla_prefill_attn_chunk, which routes each request's rows to the
# bf16 result or the fp32 state)
SPAN_KERNEL = {
    "attn_ctx": ("attn_kernel<4, false, false, 0, false, true>", "attn.hip"),
    "attn_ctx_merge": ("attn_kernel<4, false, false, 0, true, true>", "attn.hip"),
    "attn_global": ("attn_kernel<8, false, true, 2, false, false>", "attn.hip"),
    "attn_local": ("absorbed_attn_kernel", "absorbed.hip"),
    "decompress": ("decompress_kernel", "gemm.hip"),
    "gather": ("gather_kernel", "gather.hip"),
}


class KernelTimer:
    """HIP events around each launch, on the stream the kernels run on."""

    def __init__(self):
        import torch
        self.torch = torch
        self.spans = []

    @contextlib.contextmanager
    def span(self, name):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        yield
        e1.record()
        self.spans.append((name, e0, e1))

    def summary(self):
        self.torch.cuda.synchronize()
        out = {}
        for name, e0, e1 in self.spans:
            c, t = out.get(name, (0, 0.0))
            out[name] = (c + 1, t + e0.elapsed_time(e1))
        return out


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(workload, span):
    """HBM bytes per launch of a kernel from committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters (each scaled by what the same counter reads for a
    plain copy of known size); None when there is no record for this
    workload and kernel, or the kernel's source changed since the counters
    were taken."""
    if span not in SPAN_KERNEL or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        d = json.load(f).get(f"w{workload}:{span}")
    if not d or d.get("source_sha256_16") != source_hash(os.path.join(CSRC, SPAN_KERNEL[span][1])):
        return None
    return d.get("bytes_per_launch")


def _counter_rows(csv_path, counter):
    import csv
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def write_traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, workload, span, out=TRAFFIC_FILE):
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE per-dispatch counters (KiB) of one
    kernel of one workload into HBM bytes per launch, each scaled by what the
    same counter reads for the 1 GiB copy of --calibrate-copy, and store the
    record under "w<workload>:<span>" in the traffic file."""
    gib_kib = float(1 << 20)
    # the copy dispatches (the fill before them reads almost nothing)
    cal_f = [v for n, v in _counter_rows(cal_fetch_csv, "FETCH_SIZE") if v > gib_kib / 8]
    cal_w = [v for n, v in _counter_rows(cal_write_csv, "WRITE_SIZE") if v > gib_kib / 8]
    kf = gib_kib / (sum(cal_f) / len(cal_f))
    kw = gib_kib / (sum(cal_w) / len(cal_w))
    kname, src = SPAN_KERNEL[span]
    f = [v for n, v in _counter_rows(fetch_csv, "FETCH_SIZE") if kname in n]
    w = [v for n, v in _counter_rows(write_csv, "WRITE_SIZE") if kname in n]
    fetch_b = sum(f) / len(f) * 1024 * kf
    write_b = sum(w) / len(w) * 1024 * kw
    cmd = f"python3 bench.py --workload {workload} --no-sub --steps 2 --warmup 1 --no-cpu-baseline"
    rec = {"kernel": kname, "span": span, "workload": workload,
           "source_sha256_16": source_hash(os.path.join(CSRC, src)),
           "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
           "bytes_per_launch": round(fetch_b + write_b),
           "copy_scale": {"fetch": round(kf, 4), "write": round(kw, 4)},
           "launches": {"fetch": len(f), "write": len(w)},
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/f -o f -- {cmd}",
               f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/w -o w -- {cmd}",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/cf -o cf -- python3 bench.py --calibrate-copy",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/cw -o cw -- python3 bench.py --calibrate-copy",
               f"python3 bench.py --workload {workload} --traffic-span {span} --write-traffic "
               "<out>/f/f_counter_collection.csv <out>/w/w_counter_collection.csv "
               "<out>/cf/cf_counter_collection.csv <out>/cw/cw_counter_collection.csv"],
           "note": "per-dispatch counters in KiB averaged over the kernel's launches; each counter is "
                   "scaled so that the 1 GiB copy reads exactly its 1 GiB (copy_scale: the copy's FETCH_SIZE "
                   "reads half its bytes, WRITE_SIZE all of them)"}
    d = {}
    if os.path.exists(out):
        with open(out) as fh:
            d = json.load(fh)
    d[f"w{workload}:{span}"] = rec
    with open(out, "w") as fh:
        json.dump(d, fh, indent=1, sort_keys=True)
    print(json.dumps(rec))


def timed_steps(torch, run, steps, flush=None):
    """Run `steps` steps bracketed by synchronisation; returns (mean ms,
    [ms per step]). Without `flush`, events sit before each step and after
    the last. With it, `flush` runs before every step, outside that step's
    pair of events (same stream, so the step starts after it)."""
    torch.cuda.synchronize()
    if flush is None:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return ev[0].elapsed_time(ev[steps]) / max(steps, 1), per
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        flush()
        e0[i].record()
        run()
        e1[i].record()
    torch.cuda.synchronize()
    per = [e0[i].elapsed_time(e1[i]) for i in range(steps)]
    return sum(per) / max(steps, 1), per


def cache_flusher(torch, mb):
    """A callable that overwrites an `mb` MB device buffer (one fill kernel),
    so that a step's inputs are not served from the 256 MB Infinity Cache
    left warm by the previous step; None for mb = 0."""
    if mb <= 0:
        return None
    buf = torch.empty(mb << 20, dtype=torch.uint8, device="cuda")
    state = [0]

    def flush():
        state[0] ^= 1
        buf.fill_(state[0])
    return flush


def step_stats(step_ms):
    import statistics
    return {"median_ms_per_step": round(statistics.median(step_ms), 4), "min_ms_per_step": round(min(step_ms), 4)}


def gemm_reference(torch, n=8192, reps=10, zeros=False):
    """The bf16 rate of the vendor GEMM (torch.matmul, hipBLASLt) on an
    n x n x n product on this GPU: a measured ceiling for MFMA kernels at the
    clock the GPU sustains under load, beside the published peak. zeros: the
    same product on all-zero operands (the clock the GPU holds when the matrix
    cores' data does not toggle)."""
    if zeros:
        a = torch.zeros(n, n, device="cuda", dtype=torch.bfloat16)
        b = torch.zeros(n, n, device="cuda", dtype=torch.bfloat16)
    else:
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return {"op": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt){', zero operands' if zeros else ''}",
            "tflops": round(2 * n ** 3 / ms / 1e9, 1)}


def mfma_calibration(torch):
    """Sustained v_mfma_f32_32x32x16_bf16 rate on this GPU (independent
    chains on every SIMD, libmla_calib.so), or None if that library is not
    built."""
    import ctypes
    path = os.path.join(ROOT, "mla_long_context_amd", "libmla_calib.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mla_calib_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_double)]
    lib.mla_calib_mfma_bf16.restype = ctypes.c_int
    wgs = 4 * 256
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    r = ctypes.c_double(0.0)
    if lib.mla_calib_mfma_bf16(out.data_ptr(), wgs, 20000, 3, ctypes.byref(r)) != 0:
        return None
    return {"op": "independent v_mfma_f32_32x32x16_bf16 chains, 16 wavefronts per CU", "tflops": round(r.value, 1)}


def mfma_feed_calibration(torch):
    """The products of the attention loop's feed pattern without its data
    dependences (libmla_calib.so, mla_calib_mfma_fed): A operands from
    registers, from LDS at 1 KB per product, from LDS with a softmax's worth
    of independent VALU work, and from LDS with random operand bits (the
    matrix cores draw more power on toggling data, and the clock follows), at
    one workgroup per CU (one wavefront per SIMD) and two. Each rate is also
    given as a fraction of the register-operand rate at two wavefronts per
    SIMD."""
    import ctypes
    path = os.path.join(ROOT, "mla_long_context_amd", "libmla_calib.so")
    if not os.path.exists(path):
        raise SystemExit("libmla_calib.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.mla_calib_mfma_fed.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.mla_calib_mfma_fed.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(2 * cus * 256, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    names = {0: "A from registers", 1: "A from LDS, 1 KB per product", 2: "A from LDS + independent softmax VALU",
             3: "A from LDS, 1 KB per product, random operand bits"}
    rows = []
    for per_cu in (1, 2):
        for mode in (0, 1, 2, 3):
            r = ctypes.c_double(0.0)
            if lib.mla_calib_mfma_fed(out.data_ptr(), per_cu * cus, mode, 2000, 4, int(per_cu == 1),
                                      ctypes.byref(r)) != 0:
                raise SystemExit("mla_calib_mfma_fed failed")
            rows.append({"feed": names[mode], "wavefronts_per_simd": per_cu, "tflops": round(r.value, 1)})
    ref = next(x["tflops"] for x in rows if x["wavefronts_per_simd"] == 2 and x["feed"] == names[0])
    for x in rows:
        x["of_register_rate"] = round(x["tflops"] / ref, 3)
    return rows


# ---------------------------------------------------------------- the oracle on the host's cores
#
# The fp64 oracle as it stands, on a bounded sample of the workload: units of
# (request, head) for the chunked workloads (all of a request's new rows over
# all its keys, by the plain unchunked definition) and heads for the reuse
# workload (the whole document for that head, every Global row or every
# protected Local row), split over worker processes that each use one BLAS
# thread (NumPy's exp is single-threaded). The workers are forked before this
# process makes any HIP call, so they hold no GPU state, and start work only
# after the GPU timing.

_ORACLE_PROB = None
_ORACLE_DOC = None


def oracle_units(prob):
    """[(unit, algorithmic flops)] of the whole workload in a seeded order."""
    import numpy as np
    if getattr(prob, "is_reuse", False):
        Ld, T, P = int(prob.ctx_len[0]), prob.T, len(prob.prot_rows)
        units = [(("G", h), 2 * 512 * 256 * Ld + 640 * Ld * T) for h in range(prob.n_local, prob.H)]
        units += [(("L", h), 2 * 512 * 256 * Ld + 640 * Ld * P) for h in range(prob.n_local)]
    else:
        units = []
        for r in range(prob.B):
            C, E = int(prob.ctx_len[r]), int(prob.ext_len[r])
            f = 2 * 512 * 256 * (C + E) + 640 * (C * E + E * (E + 1) // 2)
            units += [((r, h), f) for h in range(prob.H)]
    order = np.random.default_rng(12345).permutation(len(units))
    return [units[i] for i in order]


def _oracle_unit(unit):
    import numpy as np
    from oracle import mla_oracle as orc
    global _ORACLE_DOC
    prob = _ORACLE_PROB
    if getattr(prob, "is_reuse", False):
        if _ORACLE_DOC is None:
            lat = orc.context_latent_f64(prob, 0, 0, int(prob.ctx_len[0]))
            _ORACLE_DOC = (lat, orc.rope_rotate(lat[:, 512:], float(prob.delta), prob.rope_base),
                           orc.bf16_to_f64(prob.W), orc.bf16_to_f64(prob.q))
        lat, k_rope, W, q = _ORACLE_DOC
        kind, h = unit
        rows = np.arange(prob.T) if kind == "G" else np.asarray(prob.prot_rows)
        kn, v = orc.decompress_head(lat[:, :512], W, prob.H, h)
        orc.attend(q[rows, h], kn, k_rope, v, prob.scale)
    else:
        r, h = unit
        orc.prefill_reference(prob, heads=[h], rows={r: np.arange(int(prob.ext_len[r]))})


def _oracle_worker(job):
    """Run units in order until the deadline; returns (flops, units, start, end)."""
    units, deadline = job
    from threadpoolctl import threadpool_limits
    flops = n = 0
    t0 = time.time()
    with threadpool_limits(1):
        for unit, f in units:
            if time.time() >= deadline:
                break
            _oracle_unit(unit)
            flops += f
            n += 1
    return flops, n, t0, time.time()


class OraclePool:
    """Worker processes for the oracle, forked now (before any HIP call)."""

    def __init__(self, prob):
        import multiprocessing as mp
        global _ORACLE_PROB
        _ORACLE_PROB = prob
        self.prob = prob
        self.affinity = len(os.sched_getaffinity(0))
        # one GPU's share of a shared host is 16 cores at most
        self.procs = max(1, min(self.affinity, 16))
        self.pool = mp.get_context("fork").Pool(self.procs)

    def run(self, budget_s=15.0):
        units = oracle_units(self.prob)
        deadline = time.time() + budget_s
        jobs = [(units[i::self.procs], deadline) for i in range(self.procs)]
        res = self.pool.map(_oracle_worker, jobs)
        self.pool.close()
        self.pool.join()
        flops = sum(r[0] for r in res)
        n = sum(r[1] for r in res)
        dt = max(r[3] for r in res) - min(r[2] for r in res)
        try:
            import numpy as np
            cfg = np.show_config(mode="dicts")
            blas = cfg.get("Build Dependencies", {}).get("blas", {}).get("name", "unknown")
        except Exception:  # pragma: no cover
            blas = "unknown"
        what = ("heads (the whole document for one head: every Global row or every protected Local row)"
                if getattr(self.prob, "is_reuse", False) else
                "(request, head) units (all of a request's new rows over all its keys for one head)")
        return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": self.procs, "kind": "oracle",
                "sample": f"{n} of {len(units)} {what} of the same workload, in a seeded order, "
                          f"{flops / 1e9:.1f} GFLOP fp64 in {dt:.1f} s; {self.procs} worker processes with one "
                          f"{blas} BLAS thread each ({self.affinity} cores in this process's affinity set)"}


def bench_append(args, torch, mla, mla_inputs):
    """mla_cache_append over every context token of the workload, written
    through the workload's own block table into a fresh pool of its dtype;
    algorithmic bytes per token: the 1152-byte bf16 record read plus the
    record written (1152 B bf16, 644 B fp8)."""
    import numpy as np
    prob = mla_inputs.make_config(args.workload)
    fp8 = prob.cache_dtype == "fp8"
    C = prob.ctx_len.astype(np.int64)
    n = int(C.sum())
    rng = np.random.default_rng(1000 + args.workload)
    src = torch.from_numpy(mla_inputs.f32_to_bf16_bits(
        rng.standard_normal((n, 576), dtype=np.float32)).view(np.int16)).view(torch.bfloat16).cuda()
    if fp8:
        pool = torch.zeros((prob.num_blocks, 41216), dtype=torch.uint8, device="cuda")
    else:
        pool = torch.zeros((prob.num_blocks, 64, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.from_numpy(np.ascontiguousarray(prob.block_table, dtype=np.int32)).cuda()
    pos0 = torch.zeros(prob.B, dtype=torch.int32, device="cuda")
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(C)]).astype(np.int32)).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cdt = mla.DTYPE_FP8_E4M3 if fp8 else mla.DTYPE_BF16

    def run():
        mla.mla_cache_append(pool, cdt, prob.num_blocks, bt, bt.shape[1], pos0, cu, prob.B, int(C.max()),
                             src, 576, status)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(args.steps, 1)
    per_tok = 1152 + (644 if fp8 else 1152)
    gbs = n * per_tok / (ms * 1e-3) / 1e9
    res = {"metric": "MLA cache append GB/s (cache write path)", "value": round(gbs, 1), "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8" if fp8 else "bf16", "data": "synthetic",
           "config": {"workload": mla_inputs.CONFIG_NAMES[args.workload] + " (context tokens appended)",
                      "tokens": n, "bytes_per_token": per_tok},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                        "kernel": "mla_cache_append", "bytes_per_launch": n * per_tok,
                        "avg_launch_ms": round(ms, 4)}}
    print(json.dumps(res))


def cpu_baseline_artifact(ap, budget_s=15.0):
    """The fp64 oracle as it stands on the artifact build: Local heads one at
    a time (decompression of the whole document for that head, then 1024
    document rows spread over it, each over its causal prefix), until about
    budget_s seconds are spent."""
    import numpy as np
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    t_dec = time.time()
    lat = np.array([orc.bf16_to_f64(ap.pool[ap.block_table[0, t // 64], t % 64]) for t in range(ap.L)])
    W = orc.bf16_to_f64(ap.W)
    rows = np.linspace(0, ap.R - 1, 1024).astype(np.int64)
    q = orc.bf16_to_f64(ap.q[rows])
    t0 = time.time()
    t_dec = t0 - t_dec
    heads = 0
    while heads < ap.n_local and (heads == 0 or time.time() - t0 < budget_s):
        orc.build_artifact(lat, q, W, ap.H, ap.n_local, ap.scale, ap.doc_rows, row_ids=rows, heads=[heads])
        heads += 1
    dt = time.time() - t0
    pos = orc.artifact_row_positions(ap.L, rows, ap.doc_rows)
    pairs = int(np.minimum(pos + 1, ap.L).sum())
    flops = heads * (2 * 512 * 256 * ap.L + 640 * pairs)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"Local heads 0..{heads - 1} (one process, {len(os.sched_getaffinity(0))} cores in its "
                      f"affinity set): decompression of the {ap.L}-token document and 1024 "
                      f"document rows spread over it (causal prefixes), {flops / 1e9:.1f} GFLOP fp64 in "
                      f"{dt:.1f} s (plus {t_dec:.1f} s decoding once, not counted); NumPy/OpenBLAS with "
                      f"{blas_threads} BLAS threads"}


def bench_artifact(args, torch, mla, mla_inputs):
    """The offline Local-head artifact build of one document (ArtifactBuilder):
    gather, decompression of the 56 Local heads, causal attention of every
    document row; TFLOP/s of algorithmic work."""
    from mla_long_context_amd.prefill import ArtifactBuilder
    t_gen = time.time()
    ap = mla_inputs.make_artifact_config()
    b = ArtifactBuilder.from_problem(ap)
    work = b.work()
    print(f"# inputs ready in {time.time() - t_gen:.1f}s: {mla_inputs.ARTIFACT_CONFIG_NAME}",
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        b.run(check=False)
    b.check()
    from mla_long_context_amd.prefill import GraphStep
    step = GraphStep(b).replay if args.graph else (lambda: b.run(check=False))
    ms, step_ms = timed_steps(torch, step, args.steps, cache_flusher(torch, args.flush_mb))
    timer = KernelTimer()
    for _ in range(args.steps):
        b.run(timer=timer, check=False)
    kern = timer.summary()
    b.check()
    flops = work["dec_flops"] + work["attn_flops"]
    tflops = flops / (ms * 1e-3) / 1e12
    per_kind = {"decompress": work["dec_flops"], "attn_causal": work["causal_attn_flops"],
                "attn_full": work["full_attn_flops"]}
    kernels = {}
    for name, (c, tot) in kern.items():
        entry = {"launches_per_step": c / args.steps, "avg_ms": round(tot / c, 4),
                 "ms_per_step": round(tot / args.steps, 4)}
        if name in per_kind:
            entry["tflops"] = round(per_kind[name] / (tot / args.steps * 1e-3) / 1e12, 2)
        else:
            entry["gbs"] = round(work["gather_bytes"] / (tot / args.steps * 1e-3) / 1e9, 1)
        kernels[name] = entry
    dom = max((k for k in kern if k in per_kind), key=lambda k: kern[k][1])
    c_ms = kern[dom][1] / kern[dom][0]
    c_unit = per_kind[dom] / (kern[dom][0] / args.steps)
    achieved = c_unit / (c_ms * 1e-3) / 1e12
    kname = {"decompress": "mla_decompress", "attn_causal": "mla_prefill_attn (causal, document rows)",
             "attn_full": "mla_prefill_attn (rows past the chunk)"}[dom]
    res = {"metric": "MLA-Off artifact build TFLOP/s (offline Local-head pass)", "value": round(tflops, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": mla_inputs.ARTIFACT_CONFIG_NAME, "heads": ap.H, "local_heads": ap.n_local,
                      "document_tokens": ap.L, "rows": ap.R, "chunk": b.S},
           "algorithmic_flop_per_step": flops,
           "document_tokens_per_s": round(ap.L / (ms * 1e-3), 1),
           "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                        "kernel": kname, "flop_per_launch": c_unit, "avg_launch_ms": round(c_ms, 4)},
           "kernels": kernels,
           "step_launch": "replay of one step captured into a HIP graph" if args.graph else "eager launches",
           "cache_flush_mb": args.flush_mb,
           "kernel_timing": "a second pass of the same number of steps, launched eagerly with HIP events around every launch"}
    res.update(step_stats(step_ms))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_artifact(ap)
    print(json.dumps(res))


KERNEL_NAMES = {
    "attn_ctx": "mla_prefill_attn_chunk (first context chunk, with the new tokens of the requests it ends)",
    "attn_ctx_merge": "mla_prefill_attn_chunk (context chunks after the first, merged into the state, "
                      "with the new tokens of the requests each ends)",
    "attn_ext": "mla_prefill_attn (causal pass)",
    "attn_last": "mla_prefill_attn_2seg (last context chunk + causal pass)",
    "decompress": "mla_decompress", "attn_global": "mla_prefill_attn (Global heads)",
    "attn_local_absorbed": "mla_absorbed_attn (protected Local rows)",
    "attn_local": "mla_prefill_attn (protected Local rows)",
    "projection": "mla_head_partition_merge", "absorb": "mla_absorb_q / mla_absorb_out",
}


def run_workload(k, prob, args, torch, steps, warmup, graph=False, min_ms=0.0):
    """Time one standard workload: `steps` timed steps (mean, median, min),
    then the same number again with events around every launch for the
    per-kernel breakdown and the dominant kernel's roofline. With min_ms,
    the step count is raised until the timed steps take at least that long
    (from a step timed after the warm-up)."""
    from mla_long_context_amd.prefill import ChunkedPrefill, GraphStep, ReusePrefill
    import mla_inputs
    reuse = bool(getattr(prob, "is_reuse", False))
    if reuse:
        kw = {} if args.split is None else {"split": args.split}
        pre = ReusePrefill(prob, chunk=args.chunk, local_path=args.local_path, **kw)
    else:
        pre = ChunkedPrefill(prob, chunk=args.chunk)
    work = pre.work()

    for _ in range(warmup):
        pre.run(check=False)
    pre.check()                      # raises if the gather saw a block id outside the pool
    # Eager launches by default; --graph replays one step captured into a
    # HIP graph instead (measured equal or slightly slower: the launches are
    # asynchronous and keep the GPU's queue full).
    step = GraphStep(pre).replay if graph else (lambda: pre.run(check=False))
    for _ in range(warmup):
        step()
    if min_ms > 0:
        est, _ = timed_steps(torch, step, 2)
        steps = max(steps, min(200, math.ceil(1.1 * min_ms / max(est, 1e-3))))   # 10% margin on the estimate

    # Timed steps for the value: events only between steps (events around
    # every launch would add a fence between kernels); the value uses the
    # mean over the K steps, the median and min per step are reported too.
    ms, step_ms = timed_steps(torch, step, steps, cache_flusher(torch, args.flush_mb))
    # The same number of steps again with events around every launch, on the
    # stream the kernels run on: per-kernel durations for the breakdown and
    # the roofline of the dominant kernel.
    timer = KernelTimer()
    torch.cuda.synchronize()
    for _ in range(steps):
        pre.run(timer=timer, check=False)
    torch.cuda.synchronize()
    kern = timer.summary()
    pre.check()

    flops = work["dec_flops"] + work["attn_flops"] + work.get("proj_flops", 0) + work.get("absorb_flops", 0)
    tflops = flops / (ms * 1e-3) / 1e12
    # algorithmic work per step of each timed kernel: flops for the MFMA
    # kernels, bytes for the HBM-bound ones
    mfma_work = {"attn_ctx": work.get("ctx_attn_flops"), "attn_ctx_merge": work.get("ctx_merge_attn_flops"),
                 "attn_ext": work.get("ext_attn_flops"), "attn_last": work.get("last_attn_flops"),
                 "decompress": work["dec_flops"], "attn_global": work.get("global_attn_flops"),
                 "attn_local": work.get("local_attn_flops"), "projection": work.get("proj_flops"),
                 "absorb": work.get("absorb_flops")}
    hbm_work = {"gather": work["gather_bytes"], "merge": work.get("merge_bytes"),
                "relocate": work.get("relocate_bytes")}
    per_step_launch = {name: c / steps for name, (c, _) in kern.items()}
    kernels = {}
    for name, (c, tot) in kern.items():
        entry = {"launches_per_step": per_step_launch[name], "avg_ms": round(tot / c, 4),
                 "ms_per_step": round(tot / steps, 4)}
        step_s = tot / steps * 1e-3           # this kernel's time per step
        if name in mfma_work:
            entry["tflops"] = round(mfma_work[name] / step_s / 1e12, 2)
            entry["mfma_frac"] = round(entry["tflops"] / PEAK_BF16_TFLOPS, 4)
        else:
            entry["gbs"] = round(hbm_work[name] / step_s / 1e9, 1)
            entry["hbm_frac"] = round(entry["gbs"] / PEAK_HBM_GBS, 4)
        kernels[name] = entry

    # the dominant kernel: the MFMA kernel with the most time per step; its
    # algorithmic flops per launch (the mean over its launches of a step,
    # which differ in a ragged batch) over its mean launch duration
    dom = max((name for name in kern if name in mfma_work), key=lambda name: kern[name][1])
    c_ms = kern[dom][1] / kern[dom][0]
    c_unit = mfma_work[dom] / per_step_launch[dom]
    achieved = c_unit / (c_ms * 1e-3) / 1e12
    span = dom
    if dom == "attn_local" and getattr(pre, "absorbed", False):
        span = "attn_local"
        kname = KERNEL_NAMES["attn_local_absorbed"]
    else:
        kname = KERNEL_NAMES[dom]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(k, span), "kernel": kname,
                "rocprof_kernel": SPAN_KERNEL.get(span, (None,))[0],
                "flop_per_launch": c_unit, "launches_per_step": per_step_launch[dom],
                "avg_launch_ms": round(c_ms, 4),
                "timing": "HIP events around each launch on the launch stream, second pass of the timed steps"}

    if reuse:
        cfg = {"workload": mla_inputs.CONFIG_NAMES[k], "heads": prob.H,
               "local_heads": pre.HL, "global_heads": pre.HG, "local_path": pre.local_path,
               "document_tokens": pre.Ldoc,
               "query_rows": pre.T, "protected_rows": pre.P, "chunk": pre.S, "split": pre.split,
               "cache": "bf16"}
    else:
        cfg = {"workload": mla_inputs.CONFIG_NAMES[k], "heads": prob.H,
               "requests": prob.B, "ctx_tokens_per_request": int(prob.ctx_len.max()),
               "ctx_tokens_total": work["ctx_tokens"],
               "new_tokens_total": work["new_tokens"], "chunk": pre.S,
               "cache": prob.cache_dtype}
    rec = {
        "value": round(tflops, 2), "unit": "TFLOP/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "config": cfg,
        "prefill_tokens_per_s": round(work["new_tokens"] / (ms * 1e-3), 1),
        "context_tokens_per_s": round(work["ctx_tokens"] / (ms * 1e-3), 1),
        "algorithmic_flop_per_step": flops,
        "mfma_roofline_frac_whole_step": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "kernels": kernels,
    }
    rec.update(step_stats(step_ms))
    del pre
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help=f"time one standard workload alone (default: workload {HEADLINE}, the headline, "
                         f"with sub-records for workloads {', '.join(map(str, SUB_WORKLOADS))})")
    ap.add_argument("--no-sub", action="store_true", help="headline only, no sub-records")
    ap.add_argument("--sub-steps", type=int, default=20,
                    help="timed steps per sub-record workload (at least 20, raised to 200 ms of timed steps)")
    ap.add_argument("--chunk", type=int, default=None, help="context chunk override (tokens)")
    ap.add_argument("--split", type=int, default=None,
                    help="reuse workload: keys per attention piece (default: the driver's)")
    ap.add_argument("--local-path", choices=["absorbed", "decompressed"], default="absorbed",
                    help="reuse workload: form of the Local heads' protected-row attention")
    ap.add_argument("--append", action="store_true",
                    help="time the cache write path instead: every context token of the workload "
                         "appended into its blocks (fp8-quantised for the fp8 workload)")
    ap.add_argument("--artifact", action="store_true",
                    help="time the offline Local-head artifact build instead (65536-token document, "
                         "56 Local heads of 64, every document row)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured into a HIP graph instead of eager launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work on the host")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="device buffer (MB) overwritten before every timed step, outside its events, "
                         "so the Infinity Cache holds nothing of the previous step (0: off)")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="only measure the MFMA rate under the attention loop's operand feed (calibration library)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB copy kernel (for HBM counter scaling)")
    ap.add_argument("--write-traffic", nargs=4, metavar="CSV",
                    help="FETCH_SIZE and WRITE_SIZE counter CSVs of a bench run, then of a "
                         "--calibrate-copy run: store the HBM-traffic record of --traffic-span for "
                         "--workload and exit")
    ap.add_argument("--traffic-span", default=None, choices=sorted(SPAN_KERNEL))
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, args.workload or HEADLINE, args.traffic_span)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs on one GPU and has no multi-GPU mode "
              "(how the path would shard is described in the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_mfma:
        import torch
        print(json.dumps({"mfma_feed": mfma_feed_calibration(torch), "mfma_sustained": mfma_calibration(torch),
                          "gemm_reference": [gemm_reference(torch), gemm_reference(torch, zeros=True)]}))
        return

    if args.calibrate_copy:
        import torch
        n = 1 << 29   # 512 Mi bf16 elements = 1 GiB
        a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 2 * n, "bytes_written": 2 * n, "launches": 3}))
        return

    import mla_inputs
    if args.append or args.artifact:
        import torch
        import mla_long_context_amd as mla
        mla.load()
        (bench_append if args.append else bench_artifact)(args, torch, mla, mla_inputs)
        return

    k = args.workload or HEADLINE
    subs = [] if (args.workload is not None or args.no_sub) else [j for j in SUB_WORKLOADS if j != k]
    # The headline's inputs, and the oracle's worker processes forked from a
    # process that has not touched the GPU yet.
    t_gen = time.time()
    prob = mla_inputs.make_config(k)
    print(f"# inputs ready in {time.time() - t_gen:.1f}s: {mla_inputs.CONFIG_NAMES[k]}",
          file=sys.stderr, flush=True)
    oracle_pool = None if args.no_cpu_baseline else OraclePool(prob)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import mla_long_context_amd as mla
    mla.load()                       # fails loudly if libmla.so is missing

    rec = run_workload(k, prob, args, torch, args.steps, args.warmup, args.graph)
    print(f"# workload {k}: {rec['ms_per_step']} ms/step, {rec['value']} TFLOP/s", file=sys.stderr, flush=True)
    res = {"metric": METRIC, "value": rec["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": rec["config"]}
    for key in ("prefill_tokens_per_s", "context_tokens_per_s", "algorithmic_flop_per_step",
                "mfma_roofline_frac_whole_step", "roofline", "kernels", "median_ms_per_step", "min_ms_per_step"):
        res[key] = rec[key]
    res["dtype_note"] = ("MFMA products in bf16 with fp32 accumulation; the fp8 cache is dequantised exactly "
                         "(fp8 codes times fp32 scales, rounded once to bf16) before the products"
                         if prob.cache_dtype == "fp8" else "MFMA products in bf16 with fp32 accumulation")
    res["step_launch"] = "replay of one step captured into a HIP graph" if args.graph else "eager launches"
    res["cache_flush_mb"] = args.flush_mb
    res["kernel_timing"] = ("a second pass of the same number of steps, launched eagerly with HIP events "
                            "around every launch")
    del prob
    if subs:
        res["workloads"] = {}
        for j in subs:
            t_gen = time.time()
            pj = mla_inputs.make_config(j)
            print(f"# inputs ready in {time.time() - t_gen:.1f}s: {mla_inputs.CONFIG_NAMES[j]}",
                  file=sys.stderr, flush=True)
            r = run_workload(j, pj, args, torch, args.sub_steps, args.warmup, args.graph, min_ms=200.0)
            print(f"# workload {j}: {r['ms_per_step']} ms/step, {r['value']} TFLOP/s", file=sys.stderr, flush=True)
            res["workloads"][str(j)] = r
            del pj
    res["gemm_reference"] = gemm_reference(torch)
    res["mfma_sustained"] = mfma_calibration(torch)
    if oracle_pool is not None:
        res["cpu_baseline"] = oracle_pool.run(args.cpu_budget)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
