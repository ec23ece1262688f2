"""End-to-end parity of the chunked prefill and the head-partitioned reuse
path on the GPU (through the C ABI) against the fp64 oracle.

Small problems are compared on every output. The five standard workloads run
at full size in the launch configuration the benchmark times; their outputs
are checked on sampled (request, row, head) entries that the oracle computes
one by one with the plain unchunked definition."""
import time

import numpy as np
import pytest
import torch

import mla_inputs as mi
from mla_long_context_amd.prefill import ChunkedPrefill, ReusePrefill
from oracle import mla_oracle as orc

from gpu_util import (FEW_KEYS, FP8_REL_L2, LSE_ABS, LSE_FEW_KEYS, bits, check_lse, check_out, f64,
                      require_gpu, say)

pytestmark = pytest.mark.gpu


def _compare_chunked(prob, pre, heads=None, rows=None, rl2=None, strict_lse=False):
    t0 = time.time()
    ref = orc.prefill_reference(prob, heads=heads, rows=rows)
    say(f"  oracle {time.time() - t0:.1f}s")
    out, lse = f64(pre.out), f64(pre.lse)
    cu = prob.cu_ext()
    H = prob.H
    heads = list(range(H)) if heads is None else list(heads)
    worst = [0.0, 0.0, 0.0]
    for r, (ro, rl) in ref.items():
        sel = np.arange(prob.ext_len[r]) if rows is None else np.asarray(rows[r])
        go = out[cu[r] + sel][:, heads]
        gl = lse[cu[r] + sel][:, heads]
        if rl2 is None:
            ma, e = check_out(go, ro, what=f"req {r} out")
        else:
            ma, e = check_out(go, ro, max_abs=1.0, rl2=rl2, what=f"req {r} out")
        n_vis = int(prob.ctx_len[r]) + sel + 1
        tol = np.where(strict_lse | (n_vis >= FEW_KEYS), LSE_ABS, LSE_FEW_KEYS)[:, None]
        le = check_lse(gl, rl, tol=tol, what=f"req {r} lse")
        worst = [max(worst[0], ma), max(worst[1], e), max(worst[2], le)]
    say(f"  worst max-abs {worst[0]:.2e} rel-L2 {worst[1]:.2e} lse {worst[2]:.2e}")
    return worst


def _run(pre):
    pre.run()
    torch.cuda.synchronize()
    assert int(pre.dev_status.item()) == 0


def test_config1_tiny_all_outputs():
    require_gpu()
    say("config 1 (tiny)")
    prob = mi.make_config(1)
    pre = ChunkedPrefill(prob)
    assert len(pre.chunks) == 2
    _run(pre)
    _compare_chunked(prob, pre, strict_lse=True)
    # twice in a row gives identical bits (no state leaks between runs)
    o1 = bits(pre.out).copy()
    _run(pre)
    assert np.array_equal(o1, bits(pre.out))


# every merge arrangement of the chunk loop: separate mla_merge_states, only
# the last merge fused into the causal pass, every merge fused with the last
# chunk and the causal pass in one launch (the default), or every merge fused
# with separate last-chunk and causal launches
@pytest.mark.parametrize("chunk,fuse,two_seg", [(64, "all", True), (100, "all", True), (4096, "all", True),
                                                (64, "all", False), (100, "all", False), (64, "none", True),
                                                (100, "final", True)])
def test_ragged_multichunk_bf16(chunk, fuse, two_seg):
    require_gpu()
    say(f"ragged bf16 chunk={chunk} fuse_merge={fuse} two_segment={two_seg}")
    prob = mi.make_problem(4, [320, 0, 64 * 9, 64], [70, 5, 300, 1], chunk, "bf16", seed=71,
                           extra_blocks=3, poison=True)
    pre = ChunkedPrefill(prob, fuse_merge=fuse, two_segment=two_seg)
    assert pre.two_seg == (two_seg and fuse == "all")
    _run(pre)
    _compare_chunked(prob, pre)


def test_ragged_multichunk_fp8():
    require_gpu()
    say("ragged fp8")
    prob = mi.make_problem(4, [64 * 11, 128, 0], [40, 257, 3], 256, "fp8", seed=72)
    pre = ChunkedPrefill(prob)
    _run(pre)
    _compare_chunked(prob, pre)
    _compare_chunked(prob, pre, rl2=FP8_REL_L2)


# key splits: one piece per chunk (5 pieces, odd merge tree), four pieces per
# chunk with a ragged last one, and the whole document as a single piece
# split / split_local: keys per Global / Local piece (one piece per chunk,
# four per chunk with a ragged last one, the whole document as one piece)
# the pieces' states merge in one pass by default; two cases keep the
# pairwise tree
@pytest.mark.parametrize("split,split_local,chunk,local,merge", [
    (2048, 8192, 256, "absorbed", "one_pass"), (64, 64, 256, "absorbed", "one_pass"),
    (64, 128, 256, "absorbed", "one_pass"), (4096, 8192, 2048, "absorbed", "one_pass"),
    (2048, 2048, 256, "decompressed", "one_pass"), (64, 64, 256, "decompressed", "one_pass"),
    (4096, 4096, 2048, "decompressed", "one_pass"), (64, 128, 256, "absorbed", "tree"),
    (64, 64, 256, "decompressed", "tree")])
def test_reuse_small_all_outputs(split, split_local, chunk, local, merge):
    require_gpu()
    say(f"reuse small split={split}/{split_local} chunk={chunk} local={local} merge={merge}")
    prob = mi.make_reuse_problem(H=8, n_local=7, L=1024 + 64, T=300, delta=4096, P=9,
                                 d_mid=256, d_model=384, chunk=chunk, seed=73)
    pre = ReusePrefill(prob, split=split, local_path=local, split_local=split_local, merge=merge)
    say(f"  {pre.n_pieces} / {pre.n_pieces_L} pieces")
    y = pre.run()
    torch.cuda.synchronize()
    ref = orc.reuse_reference(prob)
    check_out(f64(pre.glob_out), ref["O_G"], what="O_G")
    check_lse(f64(pre.lse_G), ref["lse_G"], what="lse_G")
    check_out(f64(pre.rec_out), ref["rec"], what="rec")
    check_lse(f64(pre.lse_L), ref["rec_lse"], what="rec_lse")
    ma, r = check_out(f64(y), ref["y"], what="y")
    say(f"  y max-abs {ma:.2e} rel-L2 {r:.2e}")


# several documents, each in a pool of its own at canonical positions and
# placed back to back in the request: a two-chunk, a short ragged one-chunk
# (192 keys) and a five-chunk document with a ragged tail; chunk 2048 makes
# every document a single chunk
@pytest.mark.parametrize("split,split_local,chunk,local", [
    (64, 128, 256, "absorbed"), (2048, 8192, 256, "absorbed"), (4096, 8192, 2048, "absorbed"),
    (64, 64, 256, "decompressed"), (2048, 2048, 2048, "decompressed")])
def test_multidoc_reuse_all_outputs(split, split_local, chunk, local):
    require_gpu()
    say(f"multi-document reuse split={split}/{split_local} chunk={chunk} local={local}")
    prob = mi.make_multidoc_problem(chunk=chunk)
    pre = ReusePrefill(prob, split=split, local_path=local, split_local=split_local)
    say(f"  {len(pre.docs)} documents, {len(pre.chunks)} chunks, {pre.n_pieces} / {pre.n_pieces_L} pieces")
    y = pre.run()
    torch.cuda.synchronize()
    ref = orc.reuse_reference(prob)
    check_out(f64(pre.glob_out), ref["O_G"], what="O_G")
    check_lse(f64(pre.lse_G), ref["lse_G"], what="lse_G")
    check_out(f64(pre.rec_out), ref["rec"], what="rec")
    check_lse(f64(pre.lse_L), ref["rec_lse"], what="rec_lse")
    ma, r = check_out(f64(y), ref["y"], what="y")
    say(f"  y max-abs {ma:.2e} rel-L2 {r:.2e}")


@pytest.mark.parametrize("local", ["absorbed", "decompressed"])
def test_reuse_with_empty_documents(local):
    """Degenerate documents: a request whose only document is empty (every
    recomputed row sees no key: out 0, lse -inf), and empty documents among
    non-empty ones (they contribute nothing)."""
    require_gpu()
    say(f"reuse with empty documents ({local})")
    for prob in (mi.make_reuse_problem(H=4, n_local=3, L=0, T=20, delta=4096, P=3, d_mid=128, d_model=128,
                                       chunk=256, seed=49),
                 mi.make_multidoc_problem(doc_lens=(0, 128, 0, 64), T=30, P=4, seed=50, d_mid=128, d_model=128)):
        pre = ReusePrefill(prob, split=64, split_local=64, local_path=local)
        y = pre.run()
        torch.cuda.synchronize()
        ref = orc.reuse_reference(prob)
        # 192 document keys in the second problem: the few-key lse bound
        tol = LSE_FEW_KEYS if pre.Ldoc < FEW_KEYS else LSE_ABS
        check_out(f64(pre.glob_out), ref["O_G"], what="O_G")
        check_lse(f64(pre.lse_G), ref["lse_G"], tol=tol, what="lse_G")
        check_out(f64(pre.rec_out), ref["rec"], what="rec")
        check_lse(f64(pre.lse_L), ref["rec_lse"], tol=tol, what="rec_lse")
        check_out(f64(y), ref["y"], what="y")


def test_multidoc_offsets_are_per_document():
    """Relocating every document by the first one's offset must miss the
    oracle: each document's queries are rotated by its own offset."""
    require_gpu()
    prob = mi.make_multidoc_problem(chunk=256)
    ref = orc.reuse_reference(prob)
    for d in prob.docs[1:]:
        d["delta"] = prob.docs[0]["delta"]
    pre = ReusePrefill(prob)
    pre.run()
    torch.cuda.synchronize()
    from gpu_util import rel_l2
    assert rel_l2(f64(pre.glob_out), ref["O_G"]) > 0.05


def test_reuse_without_relocation_is_caught():
    """Relocating by the wrong offset shifts every relative position; the
    Global-head outputs must then miss the oracle by far more than the bar."""
    require_gpu()
    prob = mi.make_reuse_problem(H=8, n_local=7, L=512, T=64, delta=4096, P=4,
                                 d_mid=128, d_model=128, chunk=256, seed=74)
    ref = orc.reuse_reference(prob)
    prob.delta = 0
    pre = ReusePrefill(prob)
    pre.run()
    torch.cuda.synchronize()
    from gpu_util import rel_l2
    assert rel_l2(f64(pre.glob_out), ref["O_G"]) > 0.1


# ---------------------------------------------------------------- full-size workloads

def _sample_rows(rng, E, n=6):
    pick = {0, E - 1, E // 2}
    pick |= set(int(x) for x in rng.integers(0, E, size=n))
    return np.array(sorted(pick))


@pytest.mark.parametrize("k", [2, 3, 4])
def test_full_size_workload_sampled(k):
    require_gpu()
    say(f"config {k} full size")
    t0 = time.time()
    prob = mi.make_config(k)
    say(f"  inputs {time.time() - t0:.1f}s")
    pre = ChunkedPrefill(prob)
    _run(pre)
    say(f"  gpu done {time.time() - t0:.1f}s")
    out = f64(pre.out)
    assert np.all(np.isfinite(out))
    rng = np.random.default_rng(100 + k)
    reqs = list(range(prob.B)) if prob.B <= 4 else sorted(set(rng.choice(prob.B, 3, replace=False)) | {int(np.argmax(prob.ctx_len))})
    heads = [0, prob.H - 1, int(rng.integers(1, prob.H - 1))]
    rows = {r: _sample_rows(rng, int(prob.ext_len[r])) for r in reqs}
    worst = _compare_chunked(prob, pre, heads=heads, rows=rows, strict_lse=True)
    if prob.cache_dtype == "fp8":
        assert worst[1] <= FP8_REL_L2


@pytest.mark.parametrize("local", ["absorbed", "decompressed"])
def test_full_size_reuse_sampled(local):
    require_gpu()
    say(f"config 5 full size, Local rows {local}")
    t0 = time.time()
    prob = mi.make_config(5)
    pre = ReusePrefill(prob, local_path=local)
    y = pre.run()
    torch.cuda.synchronize()
    say(f"  gpu done {time.time() - t0:.1f}s")
    assert int(pre.dev_status.item()) == 0
    rng = np.random.default_rng(105)
    # Global heads on sampled rows, protected rows for sampled Local heads,
    # by the plain definition with direct key placement
    L = int(prob.ctx_len[0])
    W = orc.bf16_to_f64(prob.W)
    lat = orc.context_latent_f64(prob, 0, 0, L)
    k_rope = orc.rope_rotate(lat[:, 512:], float(prob.delta), prob.rope_base)
    q = orc.bf16_to_f64(prob.q)
    rows = _sample_rows(rng, prob.T)
    for h in [prob.n_local, prob.H - 1]:
        kn, v = orc.decompress_head(lat[:, :512], W, prob.H, h)
        ro, rl = orc.attend(q[rows, h], kn, k_rope, v, prob.scale)
        check_out(f64(pre.glob_out)[rows, h - prob.n_local], ro, what=f"O_G head {h}")
        check_lse(f64(pre.lse_G)[rows, h - prob.n_local], rl, what=f"lse_G head {h}")
    prot = prob.prot_rows
    for h in [0, 31, prob.n_local - 1]:
        kn, v = orc.decompress_head(lat[:, :512], W, prob.H, h)
        ro, rl = orc.attend(q[prot, h], kn, k_rope, v, prob.scale)
        check_out(f64(pre.rec_out)[:, h], ro, what=f"rec head {h}")
        check_lse(f64(pre.lse_L)[:, h], rl, what=f"rec lse head {h}")
    # Equation 4 over the path's own head outputs
    O_L = orc.replace_protected(orc.bf16_to_f64(prob.art_out), f64(pre.rec_out), prot)
    ref_y = orc.head_partition_merge(O_L, f64(pre.glob_out), orc.bf16_to_f64(prob.WaL),
                                     orc.bf16_to_f64(prob.WaG), orc.bf16_to_f64(prob.Wb))
    ma, r = check_out(f64(y), ref_y, what="y")
    say(f"  y max-abs {ma:.2e} rel-L2 {r:.2e}; total {time.time() - t0:.1f}s")
