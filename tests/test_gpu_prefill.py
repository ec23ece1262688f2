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

from gpu_util import (FEW_KEYS, FP8_REL_L2, LSE_ABS, bits, check_lse, check_out, f64, kv_rounding_lse_bound,
                      relocation_lse_bound, require_gpu, say)

pytestmark = pytest.mark.gpu


def _few_key_tol(prob, r, sel, heads, exact):
    """lse tolerance per (row, head) of request r: LSE_ABS, except that rows
    seeing fewer than FEW_KEYS keys with a random kv_b_proj take the bound
    derived from their own data (kv_rounding_lse_bound), which covers the
    bf16 rounding of the decompressed keys (and of the dequantised latent of
    an fp8 cache)."""
    C, E = int(prob.ctx_len[r]), int(prob.ext_len[r])
    n_vis = C + np.asarray(sel) + 1
    tol = np.full((len(sel), len(heads)), LSE_ABS)
    few = n_vis < FEW_KEYS
    if exact or not few.any():
        return tol
    lat = orc.request_keys_f64(prob, r)
    W = orc.bf16_to_f64(prob.W)
    cu = prob.cu_ext()
    fs = np.asarray(sel)[few]
    vis = orc.causal_visible(E, C)[fs]
    for hi, h in enumerate(heads):
        q = orc.bf16_to_f64(prob.q[cu[r] + fs, h])
        b = kv_rounding_lse_bound(q, lat[:, :512], W, prob.H, h, prob.scale, vis,
                                  dequant_rounding=prob.cache_dtype == "fp8")
        tol[few, hi] = np.maximum(LSE_ABS, b)
    return tol


def _compare_chunked(prob, pre, heads=None, rows=None, rl2=None, exact=False):
    """exact: the problem's kv_b_proj is a selection matrix (and an fp8
    cache dequantises exactly), so every row is held to LSE_ABS."""
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
        le = check_lse(gl, rl, tol=_few_key_tol(prob, r, sel, heads, exact), what=f"req {r} lse")
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
    # every row sees at least 257 keys
    assert int(prob.ctx_len.min()) + 1 >= FEW_KEYS
    _compare_chunked(prob, pre)
    # twice in a row gives identical bits (no state leaks between runs)
    o1 = bits(pre.out).copy()
    _run(pre)
    assert np.array_equal(o1, bits(pre.out))


# every merge arrangement of the chunk loop: separate mla_merge_states, only
# the last merge fused into the causal pass, every merge fused with the last
# chunk and the causal pass in one launch (the default), or every merge fused
# with separate last-chunk and causal launches
# Rows of request 1 (no context, 5 new tokens) and the first rows of request
# 3 see 1..65 keys. With a selection kv_b_proj (the default here) the
# decompressed keys are exact and every row is held to the lse bar; the
# random-weight cases hold those rows to their derived bound instead.
#
# fold: each request's causal pass runs in the pass of its own last chunk
# (requests 1 and 3 end in chunk 0, requests 0 and 2 in different later
# chunks); fold=False runs them all in the loop's last pass.
@pytest.mark.parametrize("chunk,fuse,two_seg,weights,fold", [
    (64, "all", True, "selection", True), (100, "all", True, "selection", True),
    (4096, "all", True, "selection", True), (64, "all", True, "selection", False),
    (100, "all", True, "selection", False), (4096, "all", True, "selection", False),
    (64, "all", False, "selection", True), (100, "all", False, "selection", True),
    (64, "none", True, "selection", True), (100, "final", True, "selection", True),
    (100, "all", True, "normal", True), (100, "all", True, "normal", False), (64, "none", True, "normal", True)])
def test_ragged_multichunk_bf16(chunk, fuse, two_seg, weights, fold):
    require_gpu()
    say(f"ragged bf16 chunk={chunk} fuse_merge={fuse} two_segment={two_seg} weights={weights} fold={fold}")
    prob = mi.make_problem(4, [320, 0, 64 * 9, 64], [70, 5, 300, 1], chunk, "bf16", seed=71,
                           extra_blocks=3, poison=True, weights=weights)
    # the 100-token chunks gather each chunk before its decompression
    pre = ChunkedPrefill(prob, fuse_merge=fuse, two_segment=two_seg, fold_causal=fold,
                         gather_all=False if chunk == 100 else None)
    assert pre.two_seg == (two_seg and fuse == "all")
    assert pre.fold == (pre.two_seg and fold)
    _run(pre)
    _compare_chunked(prob, pre, exact=weights == "selection")


@pytest.mark.parametrize("exact,mode,gather_all", [(True, "raw", None), (False, "raw", None), (True, "dequant", None),
                                                   (False, "dequant", None), (True, "raw", False),
                                                   (True, "dequant", False)])
def test_ragged_multichunk_fp8(exact, mode, gather_all):
    """exact: selection kv_b_proj and records whose scale is 2^-6, so every
    dequantised latent and decompressed key is exact in bf16 and every row is
    held to the bar; otherwise random weights and scales, with the derived
    bound for the few-key rows. mode: the decompression reads the fp8 codes
    (raw, the default) or the gather dequantises them. gather_all=False
    gathers each chunk before its decompression instead of all at once."""
    require_gpu()
    say(f"ragged fp8 exact={exact} mode={mode} gather_all={gather_all}")
    prob = mi.make_problem(4, [64 * 11, 128, 0], [40, 257, 3], 256, "fp8", seed=72,
                           weights="selection" if exact else "normal", exact_dequant=exact)
    pre = ChunkedPrefill(prob, fp8_mode=mode, gather_all=gather_all)
    assert pre.fp8_raw == (mode == "raw")
    assert pre.gather_once == (gather_all is None)
    _run(pre)
    _compare_chunked(prob, pre, exact=exact)
    _compare_chunked(prob, pre, rl2=FP8_REL_L2, exact=exact)


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
    # 192 document keys in the second problem: a selection kv_b_proj keeps
    # the decompressed keys (and the absorbed queries) exact, so the lse bar
    # holds over so few keys
    for prob in (mi.make_reuse_problem(H=4, n_local=3, L=0, T=20, delta=4096, P=3, d_mid=128, d_model=128,
                                       chunk=256, seed=49, weights="selection"),
                 mi.make_multidoc_problem(doc_lens=(0, 128, 0, 64), T=30, P=4, seed=50, d_mid=128, d_model=128,
                                          weights="selection")):
        pre = ReusePrefill(prob, split=64, split_local=64, local_path=local)
        y = pre.run()
        torch.cuda.synchronize()
        pre.check()
        ref = orc.reuse_reference(prob)
        check_out(f64(pre.glob_out), ref["O_G"], what="O_G")
        check_lse(f64(pre.lse_G), ref["lse_G"], what="lse_G")
        check_out(f64(pre.rec_out), ref["rec"], what="rec")
        check_lse(f64(pre.lse_L), ref["rec_lse"], what="rec_lse")
        check_out(f64(y), ref["y"], what="y")


@pytest.mark.parametrize("local", ["absorbed", "decompressed"])
def test_reuse_tiny_documents(local):
    """Documents of 1 and 25 keys, and 1-, 3- and 40-key documents together.
    A selection kv_b_proj keeps every key exact, so only the relocated query
    differs from the oracle's exact rotation: the path stores it in bf16, and
    a row over so few keys keeps that rounding in its lse (over many keys it
    averages out). Outputs and y are held to the bar; lse to the bar or, if
    larger, the bound that rounding allows (relocation_lse_bound)."""
    require_gpu()
    say(f"reuse with tiny documents ({local})")
    for prob in (mi.make_reuse_problem(H=4, n_local=3, L=1, T=40, delta=4096, P=5, d_mid=128, d_model=128,
                                       chunk=256, seed=51, weights="selection"),
                 mi.make_reuse_problem(H=4, n_local=2, L=25, T=40, delta=1, P=5, d_mid=128, d_model=128,
                                       chunk=256, seed=52, weights="selection"),
                 mi.make_multidoc_problem(H=4, n_local=2, doc_lens=(1, 3, 40), T=30, P=4, seed=53, d_mid=128,
                                          d_model=128, weights="selection")):
        pre = ReusePrefill(prob, split=64, split_local=64, local_path=local)
        y = pre.run()
        torch.cuda.synchronize()
        pre.check()
        ref = orc.reuse_reference(prob)
        HL, H = prob.n_local, prob.H
        prot = np.asarray(prob.prot_rows)
        tol_g = np.stack([np.maximum(LSE_ABS, relocation_lse_bound(prob, np.arange(prob.T), h))
                          for h in range(HL, H)], axis=1)
        tol_l = np.stack([np.maximum(LSE_ABS, relocation_lse_bound(prob, prot, h)) for h in range(HL)], axis=1)
        say(f"  lse bounds: Global up to {tol_g.max():.2e}, Local up to {tol_l.max():.2e}")
        check_out(f64(pre.glob_out), ref["O_G"], what="O_G")
        check_lse(f64(pre.lse_G), ref["lse_G"], tol=tol_g, what="lse_G")
        check_out(f64(pre.rec_out), ref["rec"], what="rec")
        check_lse(f64(pre.lse_L), ref["rec_lse"], tol=tol_l, what="rec_lse")
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
    # every request (16 in the fp8 ragged workload, its first, middle and
    # last new rows plus random ones), three heads
    heads = [0, prob.H - 1, int(rng.integers(1, prob.H - 1))]
    rows = {r: _sample_rows(rng, int(prob.ext_len[r]), n=6 if prob.B <= 4 else 2) for r in range(prob.B)}
    # every sampled row sees more than FEW_KEYS keys: the lse bar applies as is
    assert int(prob.ctx_len.min()) + 1 >= FEW_KEYS
    worst = _compare_chunked(prob, pre, heads=heads, rows=rows)
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
    # y on sampled rows from the oracle's head outputs alone: three protected
    # rows (all 56 Local heads recomputed, all 8 Global heads) and three
    # unprotected ones (artifact Local rows, all 8 Global heads), each head
    # by the oracle's absorbed form over the whole document (equal to the
    # decompressed definition, pinned on the CPU), then Equation 4
    unprot = np.setdiff1d(np.arange(prob.T), prot)
    ys_p = np.sort(rng.choice(prot, 3, replace=False))
    ys_u = np.sort(rng.choice(unprot, 3, replace=False))
    ys = np.concatenate([ys_p, ys_u])
    lat_rel = np.concatenate([lat[:, :512], k_rope], axis=1)       # keys at request positions
    O_G = np.zeros((len(ys), prob.H - prob.n_local, 128))
    for gi, h in enumerate(range(prob.n_local, prob.H)):
        O_G[:, gi] = orc.attend_absorbed(q[ys, h], lat_rel, W, prob.H, h, prob.scale)[0]
    O_L = orc.bf16_to_f64(prob.art_out)[ys]
    for h in range(prob.n_local):
        O_L[:3, h] = orc.attend_absorbed(q[ys_p, h], lat_rel, W, prob.H, h, prob.scale)[0]
    ref_ys = orc.head_partition_merge(O_L, O_G, orc.bf16_to_f64(prob.WaL), orc.bf16_to_f64(prob.WaG),
                                      orc.bf16_to_f64(prob.Wb))
    ma, r = check_out(f64(y)[ys], ref_ys, what="y (oracle heads, sampled rows)")
    say(f"  y on {len(ys)} sampled rows from oracle heads: max-abs {ma:.2e} rel-L2 {r:.2e}")
    # and the projections at full size: Equation 4 over the path's own head
    # outputs, every row
    O_L = orc.replace_protected(orc.bf16_to_f64(prob.art_out), f64(pre.rec_out), prot)
    ref_y = orc.head_partition_merge(O_L, f64(pre.glob_out), orc.bf16_to_f64(prob.WaL),
                                     orc.bf16_to_f64(prob.WaG), orc.bf16_to_f64(prob.Wb))
    ma, r = check_out(f64(y), ref_y, what="y")
    say(f"  y max-abs {ma:.2e} rel-L2 {r:.2e}; total {time.time() - t0:.1f}s")


def test_out_of_range_block_raises_in_every_driver():
    """A block id outside the pool is only seen on the device: the gather
    writes zeros and sets the status word, and each driver's step raises
    instead of returning a result built from them (the word is cleared, so
    a corrected table runs clean)."""
    require_gpu()
    import mla_long_context_amd as mla
    from mla_long_context_amd.prefill import ArtifactBuilder
    prob = mi.make_problem(2, [256, 128], [40, 7], 128, "bf16", seed=76)
    prob.block_table[1, 1] = prob.num_blocks + 7
    pre = ChunkedPrefill(prob)
    with pytest.raises(mla.MlaError) as ei:
        pre.run()
    assert ei.value.code == mla._lib.MLA_ERR_OUT_OF_RANGE
    assert int(pre.dev_status.item()) == 0
    rp = mi.make_reuse_problem(H=4, n_local=3, L=256, T=20, delta=4096, P=3, d_mid=128, d_model=128,
                               chunk=128, seed=77)
    rp.block_table[0, 2] = -1
    with pytest.raises(mla.MlaError):
        ReusePrefill(rp).run()
    ap = mi.make_artifact_problem(H=4, n_local=3, L=192, extra_rows=5, doc_rows=True, chunk=128, seed=78)
    ap.block_table[0, 0] = ap.num_blocks
    with pytest.raises(mla.MlaError):
        ArtifactBuilder.from_problem(ap).run()
