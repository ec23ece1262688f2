"""Seeded random shapes through the three drivers, each against the fp64
oracle: the chunked prefill (head counts, batch sizes, context and new-token
lengths around the 64-token block and the 128-row tile, chunk sizes, bf16
and fp8 caches, the launch arrangements), head-partitioned reuse (documents,
offsets, protected rows, key splits, both Local paths, both merges), one
chunk pass with per-request last-chunk flags, and the offline artifact
build. Tolerances as in the other parity tests: rows over
fewer than 256 keys use a selection kv_b_proj (exact keys) or, with random
weights, the bound derived from their own data; reuse rows over few keys the
bound from the relocated query's rounding."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
from mla_long_context_amd.prefill import ArtifactBuilder, ChunkedPrefill, ReusePrefill
from oracle import mla_oracle as orc

from gpu_util import FP8_REL_L2, LSE_ABS, check_lse, check_out, f64, relocation_lse_bound, require_gpu, say
from test_gpu_artifact import _doc_latent, _lse_tol
from test_gpu_kernels import check_chunk_pass
from test_gpu_prefill import _compare_chunked, _run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(40))
def test_random_chunked_prefill(seed):
    require_gpu()
    rng = np.random.default_rng(1000 + seed)
    H = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 7))
    ctx = [int(rng.choice([0, 1, 63, 64, 65, int(rng.integers(0, 700)), 64 * int(rng.integers(1, 10))]))
           for _ in range(B)]
    ext = [int(rng.choice([1, 2, 31, 32, 33, 127, 128, 129, int(rng.integers(1, 300))])) for _ in range(B)]
    chunk = int(rng.choice([64, 100, 128, 256, 4096]))
    dtype = str(rng.choice(["bf16", "fp8"]))
    exact = bool(rng.integers(0, 2))
    fuse = str(rng.choice(["all", "all", "final", "none"]))
    two_seg = bool(rng.integers(0, 4) > 0)
    mode = str(rng.choice(["raw", "raw", "dequant"]))
    fold = bool(rng.integers(0, 3) > 0)
    say(f"random chunked prefill seed={seed}: H={H} ctx={ctx} ext={ext} chunk={chunk} {dtype} exact={exact} "
        f"fuse={fuse} two_seg={two_seg} fold={fold} mode={mode}")
    prob = mi.make_problem(H, ctx, ext, chunk, dtype, seed=2000 + seed, extra_blocks=int(rng.integers(0, 4)),
                           poison=True, weights="selection" if exact else "normal",
                           exact_dequant=exact and dtype == "fp8")
    pre = ChunkedPrefill(prob, fuse_merge=fuse, two_segment=two_seg, fold_causal=fold,
                         **({"fp8_mode": mode} if dtype == "fp8" else {}))
    _run(pre)
    _compare_chunked(prob, pre, exact=exact)
    if dtype == "fp8":
        _compare_chunked(prob, pre, rl2=FP8_REL_L2, exact=exact)


@pytest.mark.parametrize("seed", range(24))
def test_random_chunk_pass(seed):
    """One chunk pass (mla_prefill_attn_chunk) with random requests: lengths
    around the 64-key tile and the 32/128-row tiles, empty segments, random
    last-chunk flags, a first or a merging pass, a head range."""
    require_gpu()
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 7))
    nq = [int(rng.choice([0, 1, 31, 32, 33, 64, 65, 127, 128, 129, int(rng.integers(1, 400))])) for _ in range(B)]
    nA = [int(rng.choice([0, 1, 63, 64, 65, int(rng.integers(0, 700))])) for _ in range(B)]
    # the new tokens' keys are the rows' own, or a different count
    nB = [n if rng.integers(0, 4) else int(rng.integers(0, 300)) for n in nq]
    last = [int(rng.integers(0, 2)) for _ in range(B)]
    merge = bool(rng.integers(0, 2))
    H = int(rng.choice([1, 2, 4]))
    h0 = int(rng.integers(0, H))
    h1 = int(rng.integers(h0 + 1, H + 1))
    say(f"random chunk pass seed={seed}: nq={nq} nA={nA} nB={nB} last={last} merge={merge} heads {h0}..{h1} of {H}")
    check_chunk_pass(9100 + seed, nq, nA, nB, last, merge, H, h0, h1)


@pytest.mark.parametrize("seed", range(30))
def test_random_reuse(seed):
    require_gpu()
    rng = np.random.default_rng(5000 + seed)
    H = int(rng.choice([2, 4, 8]))
    n_local = int(rng.integers(1, H))
    L = int(rng.choice([16, 63, 64, 65, 200, int(rng.integers(16, 2000))]))
    T = int(rng.integers(1, 300))
    P = int(rng.integers(0, min(T, 20) + 1))
    chunk = int(rng.choice([64, 256, 1000, 4096]))
    split = int(rng.choice([64, 128, 512, 4096]))
    split_local = [None, 64, 256, 2048][int(rng.integers(0, 4))]
    local = str(rng.choice(["absorbed", "decompressed"]))
    merge = str(rng.choice(["one_pass", "tree"]))
    multi = bool(rng.integers(0, 4) == 0)
    if multi:
        docs = tuple(int(x) for x in rng.integers(16, 700, int(rng.integers(2, 4))))
        weights = "selection" if sum(docs) < 256 else "normal"
        prob = mi.make_multidoc_problem(H=H, n_local=n_local, doc_lens=docs, T=T, delta=4096, P=P, d_mid=128,
                                        d_model=256, chunk=chunk, seed=6000 + seed, weights=weights)
    else:
        weights = "selection" if L < 256 else "normal"
        prob = mi.make_reuse_problem(H=H, n_local=n_local, L=L, T=T, delta=int(rng.integers(0, 5000)), P=P,
                                     d_mid=128, d_model=256, chunk=chunk, seed=6000 + seed, weights=weights)
    say(f"random reuse seed={seed}: H={H} HL={n_local} L={[d['L'] for d in prob.documents()]} T={T} P={P} "
        f"chunk={chunk} split={split}/{split_local} {local} {merge} weights={weights}")
    pre = ReusePrefill(prob, split=split, local_path=local, split_local=split_local, merge=merge)
    y = pre.run()
    torch.cuda.synchronize()
    pre.check()
    ref = orc.reuse_reference(prob)
    exact = weights == "selection"
    tol_g = (np.stack([np.maximum(LSE_ABS, relocation_lse_bound(prob, np.arange(T), h)) for h in range(n_local, H)],
                      axis=1) if exact else LSE_ABS)
    check_out(f64(pre.glob_out), ref["O_G"], what="O_G")
    check_lse(f64(pre.lse_G), ref["lse_G"], tol=tol_g, what="lse_G")
    if P:
        prot = np.asarray(prob.prot_rows)
        tol_l = (np.stack([np.maximum(LSE_ABS, relocation_lse_bound(prob, prot, h)) for h in range(n_local)], axis=1)
                 if exact else LSE_ABS)
        check_out(f64(pre.rec_out), ref["rec"], what="rec")
        check_lse(f64(pre.lse_L), ref["rec_lse"], tol=tol_l, what="rec_lse")
    check_out(f64(y), ref["y"], what="y")


@pytest.mark.parametrize("seed", range(30))
def test_random_artifact_build(seed):
    require_gpu()
    rng = np.random.default_rng(7000 + seed)
    H = int(rng.choice([2, 4, 8]))
    n_local = int(rng.integers(1, H))
    L = int(rng.choice([1, 2, 63, 64, 65, 129, int(rng.integers(1, 1500))]))
    extra = int(rng.choice([0, 1, 17, 64, 130]))
    doc_rows = bool(rng.integers(0, 3) > 0)
    if not doc_rows and extra == 0:
        extra = 5
    chunk = int(rng.choice([64, 100, 256, 2048]))
    exact = bool(rng.integers(0, 2)) or L < 256
    say(f"random artifact build seed={seed}: H={H} HL={n_local} L={L} extra={extra} doc_rows={doc_rows} "
        f"chunk={chunk} exact={exact}")
    ap = mi.make_artifact_problem(H=H, n_local=n_local, L=L, extra_rows=extra, doc_rows=doc_rows, chunk=chunk,
                                  seed=8000 + seed, weights="selection" if exact else "normal")
    b = ArtifactBuilder.from_problem(ap)
    art = b.run()
    torch.cuda.synchronize()
    b.check()
    lat = _doc_latent(ap)
    out, lse = orc.build_artifact(lat, orc.bf16_to_f64(ap.q), orc.bf16_to_f64(ap.W), ap.H, ap.n_local, ap.scale,
                                  ap.doc_rows)
    check_out(f64(art.out), out, what="artifact out")
    check_lse(f64(art.lse), lse, tol=_lse_tol(ap, np.arange(out.shape[0]), list(range(ap.n_local)), lat, exact),
              what="artifact lse")
