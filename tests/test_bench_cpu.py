"""Host logic of the benchmark: the algorithmic work the headline rate
divides by, and the HBM traffic records built from rocprofv3 counters.
No GPU is used."""
import csv
import json
import os
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from mla_long_context_amd.prefill import ChunkedPrefill  # noqa: E402


def _work(ctx, ext, S, two_seg=True, H=8, cache="bf16", raw=True, fold=True):
    """ChunkedPrefill.work() of a chunk plan, without device memory: work()
    reads only the lengths, the chunk count, the head count and the launch
    arrangement."""
    pre = object.__new__(ChunkedPrefill)
    pre.prob = types.SimpleNamespace(ctx_len=np.asarray(ctx, np.int64), ext_len=np.asarray(ext, np.int64),
                                     cache_dtype=cache)
    pre.H, pre.S = H, S
    n_chunks = max((int(c) + S - 1) // S for c in ctx) if len(ctx) else 0
    pre.chunks = [None] * n_chunks
    pre.two_seg = two_seg and bool(pre.chunks)
    pre.fold = pre.two_seg and fold
    pre.fp8_raw = cache == "fp8" and raw
    return pre.work()


def _visible_pairs(ctx, ext):
    """(row, key) pairs one head attends over, counted one by one: a new row
    sees every cached context key and the new tokens up to itself (DeepSeek
    MLA -- Prefix Cache and Chunked Prefill, section 4.2)."""
    n = 0
    for C, E in zip(ctx, ext):
        for i in range(E):
            for j in range(C + E):
                n += (j < C) or (j - C <= i)
    return n


@pytest.mark.parametrize("seed", range(6))
def test_attention_work_is_the_visible_pair_count(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    ctx = [int(x) for x in rng.integers(0, 300, B)]
    ext = [int(x) for x in rng.integers(1, 40, B)]
    if max(ctx) == 0:
        ctx[0] = 1
    S = int(rng.choice([16, 64, 100, 512]))
    H = 8
    for two_seg, fold in ((True, True), (True, False), (False, False)):
        w = _work(ctx, ext, S, two_seg, H, fold=fold)
        assert w["attn_flops"] == 640 * H * _visible_pairs(ctx, ext)
        # the launches' shares partition the step's attention work
        parts = w["ctx_attn_flops"] + w["ctx_merge_attn_flops"] + w["ext_attn_flops"] + w["last_attn_flops"]
        assert parts == w["attn_flops"]
        assert w["dec_flops"] == 2 * 512 * 256 * H * (sum(ctx) + sum(ext))
        assert w["new_tokens"] == sum(ext) and w["ctx_tokens"] == sum(ctx)


def test_attention_work_by_chunk():
    # chunk c of a request holds its context keys [c S, min((c+1) S, C)); the
    # first chunk's pass, the merging passes and the last pass share them
    ctx, ext, S, H = [10, 70, 200], [3, 5, 7], 64, 2
    w = _work(ctx, ext, S, True, H, fold=False)
    per_chunk = [sum(max(0, min(S, C - c * S)) * E for C, E in zip(ctx, ext)) for c in range(4)]
    assert w["ctx_attn_flops"] == 640 * H * per_chunk[0]
    assert w["ctx_merge_attn_flops"] == 640 * H * (per_chunk[1] + per_chunk[2])
    ext_pairs = sum(E * (E + 1) // 2 for E in ext)
    assert w["last_attn_flops"] == 640 * H * (per_chunk[3] + ext_pairs)


def test_folded_causal_work_goes_to_each_request_s_last_chunk():
    # with the causal pass folded, request r's new-token pairs E(E+1)/2 are
    # counted in the pass of its last chunk max(ceil(C/S) - 1, 0): requests
    # of 0 and 10 context tokens end in chunk 0, the one of 70 in chunk 1,
    # the one of 200 in chunk 3
    ctx, ext, S, H = [10, 70, 200, 0], [3, 5, 7, 4], 64, 2
    w = _work(ctx, ext, S, True, H)
    per_chunk = [sum(max(0, min(S, C - c * S)) * E for C, E in zip(ctx, ext)) for c in range(4)]
    causal = [E * (E + 1) // 2 for E in ext]
    assert w["ctx_attn_flops"] == 640 * H * (per_chunk[0] + causal[0] + causal[3])
    assert w["ctx_merge_attn_flops"] == 640 * H * (sum(per_chunk[1:]) + causal[1] + causal[2])
    assert w["last_attn_flops"] == 0 and w["ext_attn_flops"] == 0
    # 70 tokens is two chunks of 64: request 1 ends in chunk 1, a merging pass
    assert _work([70], [5], 64, True, H)["ctx_merge_attn_flops"] == 640 * H * (6 * 5 + 15)


def test_dsv3_workload_flops():
    # 128 heads, 4 requests of 8192 cached and 1024 new tokens, chunk 4096
    w = _work([8192] * 4, [1024] * 4, 4096, True, 128)
    assert w["dec_flops"] == 2 * 512 * 256 * 128 * 4 * 9216 == 1_236_950_581_248
    assert w["attn_flops"] == 640 * 128 * 4 * (8192 * 1024 + 1024 * 1025 // 2) == 2_920_745_533_440
    assert w["dec_flops"] + w["attn_flops"] == 4_157_696_114_688


def test_gather_bytes_per_token():
    # bf16 records move 1152 bytes in and out; fp8 records 644 in (512 codes,
    # 128 rope bytes, a 4-byte scale) and 644 out as raw codes, or 1152 out
    # when widened to bf16
    assert _work([100], [4], 64, cache="bf16")["gather_bytes"] == 100 * 2304
    assert _work([100], [4], 64, cache="fp8", raw=True)["gather_bytes"] == 100 * (644 + 644)
    assert _work([100], [4], 64, cache="fp8", raw=False)["gather_bytes"] == 100 * (644 + 1152)


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for k, c, v in rows:
            wr.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_record_scaling_and_staleness(tmp_path, monkeypatch):
    kname = bench.SPAN_KERNEL["attn_ctx_merge"][0]
    gib_kib = 1 << 20
    # the copy: its fill dispatch reads almost nothing; FETCH_SIZE reads half
    # the copied GiB, WRITE_SIZE all of it
    _counter_csv(tmp_path / "cf.csv", [("fill", "FETCH_SIZE", 10)] + [("copy", "FETCH_SIZE", gib_kib // 2)] * 3)
    _counter_csv(tmp_path / "cw.csv", [("fill", "WRITE_SIZE", gib_kib)] + [("copy", "WRITE_SIZE", gib_kib)] * 3)
    # two dispatches of the kernel, and one of another kernel that must be ignored
    _counter_csv(tmp_path / "f.csv", [(f"void {kname}(AttnArgs)", "FETCH_SIZE", 1000),
                                      (f"void {kname}(AttnArgs)", "FETCH_SIZE", 3000),
                                      ("void gather_kernel<true, true>", "FETCH_SIZE", 99999)])
    _counter_csv(tmp_path / "w.csv", [(f"void {kname}(AttnArgs)", "WRITE_SIZE", 500),
                                      (f"void {kname}(AttnArgs)", "WRITE_SIZE", 500)])
    out = tmp_path / "traffic.json"
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                        str(tmp_path / "cw.csv"), 4, "attn_ctx_merge", out=str(out))
    rec = json.load(open(out))["w4:attn_ctx_merge"]
    assert rec["fetch_bytes_per_launch"] == 2000 * 1024 * 2
    assert rec["write_bytes_per_launch"] == 500 * 1024
    assert rec["bytes_per_launch"] == 2000 * 1024 * 2 + 500 * 1024
    assert rec["launches"] == {"fetch": 2, "write": 2}
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.traffic_for(4, "attn_ctx_merge") == rec["bytes_per_launch"]
    assert bench.traffic_for(2, "attn_ctx_merge") is None          # no record for that workload
    d = json.load(open(out))
    d["w4:attn_ctx_merge"]["source_sha256_16"] = "0" * 16        # the kernel source changed since
    json.dump(d, open(out, "w"))
    assert bench.traffic_for(4, "attn_ctx_merge") is None


def _reuse_work(absorbed, merge="one_pass", n_pieces=64, n_pieces_L=36):
    """ReusePrefill.work() of the head-partitioned reuse workload's plan: 64
    heads (56 Local, 8 Global), a 262144-token document, 512 query rows, 64
    protected rows, W_a 8192 -> 2048, W_b 2048 -> 4096."""
    from mla_long_context_amd.prefill import ReusePrefill
    pre = object.__new__(ReusePrefill)
    pre.H, pre.HL, pre.HG, pre.T, pre.P, pre.Ldoc = 64, 56, 8, 512, 64, 262144
    pre.n_pieces, pre.n_pieces_L = n_pieces, n_pieces_L
    pre.absorbed, pre.merge_mode = absorbed, merge
    pre.d_mid, pre.d_model = 2048, 4096
    pre.docs = [None]
    return pre.work()


def test_reuse_workload_flops():
    # decompressed Local rows: every head decompressed over the document,
    # 640 flop per (row, key, head) for the 512 Global rows x 8 heads and the
    # 64 protected rows x 56 Local heads, and the two projections of
    # Equation 4 (RedKnot-MLA, section 2)
    w = _reuse_work(absorbed=False)
    L = 262144
    assert w["dec_flops"] == 2 * 512 * 256 * 64 * L
    assert w["global_attn_flops"] == 640 * L * 512 * 8
    assert w["local_attn_flops"] == 640 * L * 64 * 56
    assert w["proj_flops"] == 2 * 512 * (64 * 128 * 2048 + 2048 * 4096)
    total = w["dec_flops"] + w["attn_flops"] + w["proj_flops"]
    assert abs(total - 5.71e12) < 0.01e12
    # absorbed Local rows: only the Global heads are decompressed; a Local
    # (row, key, head) costs 2*576 for the scores over the latent and 2*512
    # for the latent-space values; the query absorption and the W_UV product
    # cost 2*128*512 each per (row, head)
    a = _reuse_work(absorbed=True)
    assert a["dec_flops"] == 2 * 512 * 256 * 8 * L
    assert a["local_attn_flops"] == (2 * 576 + 2 * 512) * L * 64 * 56
    assert a["absorb_flops"] == 2 * (2 * 128 * 512) * 64 * 56
    assert a["global_attn_flops"] == w["global_attn_flops"]


def test_oracle_units_cover_the_workload_once():
    # the cpu baseline's units are (request, head) pairs of the tiny workload,
    # each carrying its share of the same algorithmic count as the GPU's value
    import mla_inputs as mi
    prob = mi.make_config(1)
    units = bench.oracle_units(prob)
    assert sorted(u for u, _ in units) == [(r, h) for r in range(prob.B) for h in range(prob.H)]
    w = _work(list(prob.ctx_len), list(prob.ext_len), prob.chunk, True, prob.H)
    assert sum(f for _, f in units) == w["dec_flops"] + w["attn_flops"]
    assert units == bench.oracle_units(prob)            # seeded order


def test_oracle_pool_reports_the_rate_of_the_units_it_ran():
    import mla_inputs as mi
    prob = mi.make_config(1)
    pool = bench.OraclePool(prob)
    rec = pool.run(budget_s=3.0)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s" and rec["value"] > 0
    assert rec["cores"] == min(len(os.sched_getaffinity(0)), 16)
    assert f"of {prob.B * prob.H} " in rec["sample"]
