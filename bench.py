#!/usr/bin/env python3
"""Benchmark of MLA chunked prefill on one MI355X.

Workload (default): DeepSeek-V3 geometry, one layer, 128 heads, 4 requests x
(8192 cached context tokens + 1024 new tokens), 64-token blocks in a shuffled
pool, context chunk 4096, bf16 cache. A step is one pass of the whole path:
per context chunk gather -> kv_b_proj decompression -> attention -> LSE merge
into the running state; the last chunk's attention also covers the new
tokens' keys (decompressed beside the chunk's, causal) and writes the result.
Inputs are seeded synthetic data resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]

Prints one JSON line: TFLOP/s of algorithmic work (2*512*256 flop per
decompressed (token, head), 640 flop per visible (row, key, head)) over the
timed steps (eager launches; --graph replays one step captured into a HIP
graph), prefill tokens/s, the roofline of the dominant kernel (per-launch
duration from HIP events on the launch stream, taken in a second pass of the
same number of steps, since events between launches add fences to the step),
and the fp64 CPU oracle timed on a bounded sample on this host.

    python bench.py --workload {1..5}   # the other standard workloads
    python bench.py --append            # the cache write path
    python bench.py --artifact          # the offline Local-head artifact build
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MLA chunked-prefill TFLOP/s + prefill tokens/s; % of MFMA/HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_2seg_dsv3_hbm_traffic.json")


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


def traffic_for(kernel_src):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, scaled by a plain copy's counter reading; None when absent or
    when the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        d = json.load(f)
    if d.get("source_sha256_16") != source_hash(kernel_src):
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


def write_traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, out=TRAFFIC_FILE):
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE per-dispatch counters (KiB) of the
    two-segment attention launches (the dominant kernel of the dsv3 workload)
    into HBM bytes per launch, each scaled by what
    the same counter reads for the 1 GiB copy of --calibrate-copy."""
    gib_kib = float(1 << 20)
    # the copy dispatches (the fill before them reads almost nothing)
    cal_f = [v for n, v in _counter_rows(cal_fetch_csv, "FETCH_SIZE") if v > gib_kib / 8]
    cal_w = [v for n, v in _counter_rows(cal_write_csv, "WRITE_SIZE") if v > gib_kib / 8]
    kf = gib_kib / (sum(cal_f) / len(cal_f))
    kw = gib_kib / (sum(cal_w) / len(cal_w))
    # the two-segment pass (last chunk + new tokens; bf16 out, merged)
    ctx = lambda n: "attn_kernel<4, false, false, 0, true, true>" in n
    f = [v for n, v in _counter_rows(fetch_csv, "FETCH_SIZE") if ctx(n)]
    w = [v for n, v in _counter_rows(write_csv, "WRITE_SIZE") if ctx(n)]
    fetch_b = sum(f) / len(f) * 1024 * kf
    write_b = sum(w) / len(w) * 1024 * kw
    d = {"kernel": "mla_prefill_attn_2seg (second context chunk + causal pass), 4 x (8192 ctx + 1024 new), "
                   "H=128, chunk 4096",
         "source_sha256_16": source_hash(os.path.join(ROOT, "mla_long_context_amd", "csrc", "attn.hip")),
         "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
         "bytes_per_launch": round(fetch_b + write_b),
         "copy_scale": {"fetch": round(kf, 4), "write": round(kw, 4)},
         "launches": {"fetch": len(f), "write": len(w)},
         "commands": [
             "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/f -o f -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
             "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/w -o w -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
             "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/cf -o cf -- python3 bench.py --calibrate-copy",
             "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/cw -o cw -- python3 bench.py --calibrate-copy",
             "python3 bench.py --write-traffic <out>/f/f_counter_collection.csv <out>/w/w_counter_collection.csv "
             "<out>/cf/cf_counter_collection.csv <out>/cw/cw_counter_collection.csv"],
         "note": "per-dispatch counters in KiB, averaged over the two-segment attention launches; the 1 GiB "
                 "copy reads FETCH_SIZE x 1/2 and WRITE_SIZE x 1, hence the scales"}
    with open(out, "w") as fh:
        json.dump(d, fh, indent=1)
    print(json.dumps(d))


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


def gemm_reference(torch, n=8192, reps=10):
    """The bf16 rate of the vendor GEMM (torch.matmul, hipBLASLt) on an
    n x n x n product on this GPU: a measured ceiling for MFMA kernels at the
    clock the GPU sustains under load, beside the published peak."""
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
    return {"op": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt)", "tflops": round(2 * n ** 3 / ms / 1e9, 1)}


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


def cpu_baseline(prob, budget_s=15.0):
    """The fp64 oracle as it stands, on request 0 of the same workload, one
    head at a time, until about budget_s seconds of host work are spent."""
    import numpy as np
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    C, E = int(prob.ctx_len[0]), int(prob.ext_len[0])
    per_head = 2 * 512 * 256 * (C + E) + 640 * (C * E + E * (E + 1) // 2)
    heads = 0
    t0 = time.time()
    while heads < prob.H and time.time() - t0 < budget_s:
        orc.prefill_reference(prob, heads=[heads], rows={0: np.arange(E)})
        heads += 1
    dt = time.time() - t0
    flops = per_head * heads
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"request 0 (C={C}, E={E}), heads 0..{heads - 1} of {prob.H}, all {E} new rows: "
                      f"{flops / 1e9:.1f} GFLOP fp64 in {dt:.1f} s; NumPy/OpenBLAS with "
                      f"{blas_threads} BLAS threads (exp single-threaded)"}


def cpu_baseline_reuse(prob, budget_s=15.0):
    """The fp64 oracle as it stands on the reuse workload: Global heads one
    at a time (decompression of the whole document for that head, then all
    query rows against it), until about budget_s seconds are spent."""
    import numpy as np
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    H, HL, T = prob.H, prob.n_local, prob.T
    Ld = int(prob.ctx_len[0])
    t_dec = time.time()
    W = orc.bf16_to_f64(prob.W)
    lat = orc.context_latent_f64(prob, 0, 0, Ld)
    k_rope = orc.rope_rotate(lat[:, 512:], float(prob.delta), prob.rope_base)
    q = orc.bf16_to_f64(prob.q)
    t0 = time.time()
    t_dec = t0 - t_dec
    heads = 0
    while HL + heads < H and (heads == 0 or time.time() - t0 < budget_s):
        h = HL + heads
        kn, v = orc.decompress_head(lat[:, :512], W, H, h)
        orc.attend(q[:, h], kn, k_rope, v, prob.scale)
        heads += 1
    dt = time.time() - t0
    flops = heads * (2 * 512 * 256 * Ld + 640 * Ld * T)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"Global heads {HL}..{HL + heads - 1}: decompression of the {Ld}-token document "
                      f"and all {T} query rows, {flops / 1e9:.1f} GFLOP fp64 in {dt:.1f} s (plus {t_dec:.1f} s "
                      f"decoding the document once, not counted); NumPy/OpenBLAS with {blas_threads} BLAS threads"}


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
            "sample": f"Local heads 0..{heads - 1}: decompression of the {ap.L}-token document and 1024 "
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
        b.run()
    torch.cuda.synchronize()
    assert int(b.dev_status.item()) == 0
    from mla_long_context_amd.prefill import GraphStep
    step = GraphStep(b).replay if args.graph else b.run
    ms, step_ms = timed_steps(torch, step, args.steps, cache_flusher(torch, args.flush_mb))
    timer = KernelTimer()
    for _ in range(args.steps):
        b.run(timer=timer)
    kern = timer.summary()
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
           "cache_flush_mb": args.flush_mb,
           "kernel_timing": "a second pass of the same number of steps, launched eagerly with HIP events around every launch"}
    res.update(step_stats(step_ms))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_artifact(ap)
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="standard workload number; 2 (the default) is the headline line")
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
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="device buffer (MB) overwritten before every timed step, outside its events, "
                         "so the Infinity Cache holds nothing of the previous step (0: off)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB copy kernel (for HBM counter scaling)")
    ap.add_argument("--write-traffic", nargs=4, metavar="CSV",
                    help="FETCH_SIZE and WRITE_SIZE counter CSVs of a bench run, then of a "
                         "--calibrate-copy run: write the HBM-traffic record and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only; the prefill path has no multi-GPU mode. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.calibrate_copy:
        n = 1 << 29   # 512 Mi bf16 elements = 1 GiB
        a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 2 * n, "bytes_written": 2 * n, "launches": 3}))
        return

    import mla_inputs
    import mla_long_context_amd as mla
    from mla_long_context_amd.prefill import ChunkedPrefill, GraphStep, ReusePrefill

    if args.append:
        bench_append(args, torch, mla, mla_inputs)
        return
    if args.artifact:
        mla.load()
        bench_artifact(args, torch, mla, mla_inputs)
        return

    mla.load()                       # fails loudly if libmla.so is missing
    t_gen = time.time()
    prob = mla_inputs.make_config(args.workload)
    reuse = bool(getattr(prob, "is_reuse", False))
    if reuse:
        kw = {} if args.split is None else {"split": args.split}
        pre = ReusePrefill(prob, chunk=args.chunk, local_path=args.local_path, **kw)
    else:
        pre = ChunkedPrefill(prob, chunk=args.chunk)
    work = pre.work()
    print(f"# inputs ready in {time.time() - t_gen:.1f}s: {mla_inputs.CONFIG_NAMES[args.workload]}",
          file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        pre.run()
    torch.cuda.synchronize()
    assert int(pre.dev_status.item()) == 0, "gather reported an out-of-range block"
    # Eager launches by default; --graph replays one step captured into a
    # HIP graph instead (measured equal or slightly slower: the launches are
    # asynchronous and keep the GPU's queue full).
    step = GraphStep(pre).replay if args.graph else pre.run
    for _ in range(args.warmup):
        step()

    # Timed steps for the headline value: events only between steps (events
    # around every launch would add a fence between kernels); the value uses
    # the mean over the K steps, the median and min per step are reported too.
    ms, step_ms = timed_steps(torch, step, args.steps, cache_flusher(torch, args.flush_mb))
    # The same number of steps again with events around every launch, on the
    # stream the kernels run on: per-kernel durations for the breakdown and
    # the roofline of the dominant kernel.
    timer = KernelTimer()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        pre.run(timer=timer)
    torch.cuda.synchronize()
    kern = timer.summary()

    flops = work["dec_flops"] + work["attn_flops"] + work.get("proj_flops", 0) + work.get("absorb_flops", 0)
    tflops = flops / (ms * 1e-3) / 1e12
    # algorithmic work per step of each timed kernel: flops for the MFMA
    # kernels, bytes for the HBM-bound ones
    mfma_work = {"attn_ctx": work.get("ctx_attn_flops"), "attn_ext": work.get("ext_attn_flops"),
                 "attn_last": work.get("last_attn_flops"),
                 "decompress": work["dec_flops"], "attn_global": work.get("global_attn_flops"),
                 "attn_local": work.get("local_attn_flops"), "projection": work.get("proj_flops"),
                 "absorb": work.get("absorb_flops")}
    hbm_work = {"gather": work["gather_bytes"], "merge": work.get("merge_bytes"),
                "relocate": work.get("relocate_bytes")}
    per_step_launch = {k: c / args.steps for k, (c, _) in kern.items()}
    kernels = {}
    for name, (c, tot) in kern.items():
        avg = tot / c
        entry = {"launches_per_step": per_step_launch[name], "avg_ms": round(avg, 4),
                 "ms_per_step": round(tot / args.steps, 4)}
        step_s = tot / args.steps * 1e-3           # this kernel's time per step
        if name in mfma_work:
            entry["tflops"] = round(mfma_work[name] / step_s / 1e12, 2)
        else:
            entry["gbs"] = round(hbm_work[name] / step_s / 1e9, 1)
        kernels[name] = entry

    # the dominant kernel: the MFMA kernel with the most time per step
    dom = max((k for k in kern if k in mfma_work), key=lambda k: kern[k][1])
    c_ms = kern[dom][1] / kern[dom][0]
    c_unit = mfma_work[dom] / per_step_launch[dom]
    achieved = c_unit / (c_ms * 1e-3) / 1e12
    traffic = None
    if dom == "attn_last" and args.workload == 2:   # the workload the counter record was taken on
        traffic = traffic_for(os.path.join(ROOT, "mla_long_context_amd", "csrc", "attn.hip"))
    kname = {"attn_ctx": "mla_prefill_attn (context pass)", "attn_ext": "mla_prefill_attn (causal pass)",
             "attn_last": "mla_prefill_attn_2seg (last context chunk + causal pass)",
             "decompress": "mla_decompress", "attn_global": "mla_prefill_attn (Global heads)",
             "attn_local": ("mla_absorbed_attn (protected Local rows)" if getattr(pre, "absorbed", False)
                            else "mla_prefill_attn (protected Local rows)"),
             "projection": "mla_head_partition_merge",
             "absorb": "mla_absorb_q / mla_absorb_out"}[dom]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": kname,
                "flop_per_launch": c_unit, "avg_launch_ms": round(c_ms, 4)}

    if reuse:
        cfg = {"workload": mla_inputs.CONFIG_NAMES[args.workload], "heads": prob.H,
               "local_heads": pre.HL, "global_heads": pre.HG, "local_path": pre.local_path,
               "document_tokens": pre.Ldoc,
               "query_rows": pre.T, "protected_rows": pre.P, "chunk": pre.S, "split": pre.split,
               "cache": "bf16"}
    else:
        cfg = {"workload": mla_inputs.CONFIG_NAMES[args.workload], "heads": prob.H,
               "requests": prob.B, "ctx_tokens_per_request": int(prob.ctx_len.max()),
               "new_tokens_total": work["new_tokens"], "chunk": pre.S,
               "cache": prob.cache_dtype}
    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": cfg,
        "prefill_tokens_per_s": round(work["new_tokens"] / (ms * 1e-3), 1),
        "context_tokens_per_s": round(work["ctx_tokens"] / (ms * 1e-3), 1),
        "algorithmic_flop_per_step": flops,
        "mfma_roofline_frac_whole_step": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "kernels": kernels,
        "step_launch": "replay of one step captured into a HIP graph" if args.graph else "eager launches",
        "cache_flush_mb": args.flush_mb,
        "kernel_timing": "a second pass of the same number of steps, launched eagerly with HIP events around every launch",
    }
    res.update(step_stats(step_ms))
    res["gemm_reference"] = gemm_reference(torch)
    res["mfma_sustained"] = mfma_calibration(torch)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_reuse(prob) if reuse else cpu_baseline(prob)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
