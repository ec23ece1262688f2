"""Offline Local-head artifact (MLA-Off) on the GPU against the fp64 oracle:
the build itself (document rows causal, rows after the document, one or
several key chunks), the artifact fed to the reuse path (Equation 4 then
equals full recomputation), and the fallback to full recomputation when the
artifact's description does not match the request."""
import dataclasses

import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_long_context_amd as mla
from mla_long_context_amd.prefill import ArtifactBuilder, ReusePrefill, artifact_meta
from oracle import mla_oracle as orc

from gpu_util import FEW_KEYS, LSE_ABS, check_lse, check_out, f64, kv_rounding_lse_bound, require_gpu, say

pytestmark = pytest.mark.gpu


def _doc_latent(ap):
    return np.array([orc.bf16_to_f64(ap.pool[ap.block_table[0, t // 64], t % 64]) for t in range(ap.L)])


def _lse_tol(ap, row_ids, heads, latent, exact):
    """LSE_ABS, except rows that see fewer than FEW_KEYS document keys with a
    random kv_b_proj: those take the bound derived from their own data
    (kv_rounding_lse_bound). With a selection kv_b_proj (exact) every row
    is held to LSE_ABS."""
    row_ids = np.asarray(row_ids)
    pos = orc.artifact_row_positions(ap.L, row_ids, ap.doc_rows)
    nkeys = np.minimum(pos + 1, ap.L)
    tol = np.full((len(row_ids), len(heads)), LSE_ABS)
    few = nkeys < FEW_KEYS
    if exact or not few.any():
        return tol
    W = orc.bf16_to_f64(ap.W)
    vis = np.arange(ap.L)[None, :] <= pos[few][:, None]
    for j, h in enumerate(heads):
        q = orc.bf16_to_f64(ap.q[row_ids[few], h])
        tol[few, j] = np.maximum(LSE_ABS, kv_rounding_lse_bound(q, latent[:, :512], W, ap.H, h, ap.scale, vis))
    return tol


# document rows with several chunks and a ragged last one (1088 = 4 x 256 + 64)
# plus 50 rows after the document; one chunk for the whole document; only rows
# after the document; a chunk that is not a multiple of the block size
@pytest.mark.parametrize("doc_rows,chunk,extra", [(True, 256, 50), (True, 2048, 50), (False, 256, 77),
                                                  (True, 300, 0)])
def test_artifact_build_parity(doc_rows, chunk, extra):
    require_gpu()
    say(f"artifact build doc_rows={doc_rows} chunk={chunk} extra={extra}")
    # document rows see 1..L keys: a selection kv_b_proj keeps the
    # decompressed keys exact so every row is held to the lse bar
    ap = mi.make_artifact_problem(H=8, n_local=7, L=1088, extra_rows=extra, doc_rows=doc_rows, chunk=chunk,
                                  seed=44, weights="selection")
    b = ArtifactBuilder.from_problem(ap)
    art = b.run()
    torch.cuda.synchronize()
    b.check()
    out, lse = orc.build_artifact(_doc_latent(ap), orc.bf16_to_f64(ap.q), orc.bf16_to_f64(ap.W), ap.H,
                                  ap.n_local, ap.scale, ap.doc_rows)
    ma, r = check_out(f64(art.out), out, what="artifact out")
    e = check_lse(f64(art.lse), lse, tol=LSE_ABS, what="artifact lse")
    say(f"  out max-abs {ma:.2e} rel-L2 {r:.2e}, lse max-abs {e:.2e}")
    assert art.meta.token_hash == orc.artifact_token_hash(ap.tokens)
    assert art.meta.n_tokens == ap.L and art.meta.generation == ap.generation


def test_artifact_of_an_empty_document():
    """No document keys: every row's Local-head state is (0, -inf), the
    identity of the merge."""
    require_gpu()
    ap = mi.make_artifact_problem(H=4, n_local=3, L=64, extra_rows=40, doc_rows=False, chunk=64, seed=48)
    b = ArtifactBuilder(ap.pool, ap.block_table, 0, ap.q, ap.W, ap.H, ap.n_local, ap.scale, doc_rows=False,
                        chunk=64, tokens=ap.tokens[:0], generation=1)
    art = b.run()
    torch.cuda.synchronize()
    assert tuple(art.out.shape) == (40, 3, 128) and tuple(art.lse.shape) == (40, 3)
    assert np.all(f64(art.out) == 0.0)
    assert np.all(np.isneginf(f64(art.lse)))
    assert art.meta.n_tokens == 0


def _request_meta(prob, tokens, generation, **kw):
    m = artifact_meta(tokens, generation, prob.H, prob.n_local, prob.rope_base)
    for k, v in kw.items():
        setattr(m, k, v)
    return m


def _built_for_request(prob, tokens, generation, chunk=256):
    """The artifact of the request's T rows: their queries moved into the
    document's canonical frame (rows after the document), built offline."""
    q = mi_bf16(prob.q)
    q_c = torch.empty_like(q)
    mla.mla_rope_relocate_q(q, q_c, prob.H * 192, prob.T, prob.H, prob.delta, prob.rope_base)
    b = ArtifactBuilder(prob.pool, prob.block_table, int(prob.ctx_len[0]), q_c, prob.W, prob.H, prob.n_local,
                        prob.scale, doc_rows=False, chunk=chunk, tokens=tokens, generation=generation,
                        rope_base=prob.rope_base)
    return b.run()


def mi_bf16(bits_arr):
    return torch.from_numpy(np.ascontiguousarray(bits_arr).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("local", ["absorbed", "decompressed"])
def test_built_artifact_makes_reuse_equal_full_recompute(local):
    """Equation 4 is exact under full recomputation: with the artifact of the
    request's own rows (unchanged context), the reuse output equals the
    oracle's full recomputation of every Local row."""
    require_gpu()
    say(f"built artifact -> reuse ({local})")
    prob = mi.make_reuse_problem(H=8, n_local=7, L=1024 + 64, T=300, delta=4096, P=9,
                                 d_mid=256, d_model=384, chunk=256, seed=45)
    tokens = mi.document_tokens(int(prob.ctx_len[0]), seed=45)
    art = _built_for_request(prob, tokens, generation=5)
    pre = ReusePrefill(prob, split=256, split_local=512, local_path=local, artifact=art,
                       request=_request_meta(prob, tokens, 5))
    assert pre.fallback is None
    y = pre.run()
    torch.cuda.synchronize()
    full = orc.reuse_reference(dataclasses.replace(prob, prot_rows=np.arange(prob.T, dtype=np.int32)))
    check_out(f64(art.out), full["rec"], what="artifact rows")
    ma, r = check_out(f64(y), full["y"], what="y")
    say(f"  y max-abs {ma:.2e} rel-L2 {r:.2e}")


@pytest.mark.parametrize("case", ["stale", "tokens", "layer", "profile"])
def test_invalid_artifact_falls_back_to_full_recompute(case):
    """A stale, mismatched or incomplete artifact is never read (its values
    here are NaN): every Local row is recomputed and y equals the full
    recomputation."""
    require_gpu()
    say(f"artifact fallback: {case}")
    prob = mi.make_reuse_problem(H=8, n_local=7, L=512 + 64, T=120, delta=4096, P=5,
                                 d_mid=128, d_model=256, chunk=256, seed=46)
    tokens = mi.document_tokens(int(prob.ctx_len[0]), seed=46)
    art = _built_for_request(prob, tokens, generation=2)
    art.out.fill_(float("nan"))
    if case == "stale":
        req = _request_meta(prob, tokens, 3)
    elif case == "tokens":
        t2 = tokens.copy(); t2[100] += 1
        req = _request_meta(prob, t2, 2)
    elif case == "layer":
        req = _request_meta(prob, tokens, 2, layer_mask=0b11)
    else:
        req = _request_meta(prob, tokens, 2, n_local=6)
    pre = ReusePrefill(prob, artifact=art, request=req)
    expect = {"stale": "stale generation", "tokens": "token mismatch", "layer": "missing layer",
              "profile": "profile mismatch"}[case]
    assert pre.fallback == expect
    assert pre.P == prob.T and pre.local_path == "decompressed"
    y = pre.run()
    torch.cuda.synchronize()
    full = orc.reuse_reference(dataclasses.replace(prob, prot_rows=np.arange(prob.T, dtype=np.int32)))
    ma, r = check_out(f64(y), full["y"], what="y")
    say(f"  y max-abs {ma:.2e} rel-L2 {r:.2e}")


def test_artifact_full_size_sampled():
    """The benchmark's build (65536-token document, 64 heads of which 56
    Local, every document row, one chunk) on sampled rows and heads."""
    require_gpu()
    say("artifact build, full size")
    ap = mi.make_artifact_config()
    b = ArtifactBuilder.from_problem(ap)
    art = b.run()
    torch.cuda.synchronize()
    assert int(b.dev_status.item()) == 0
    got_o, got_l = f64(art.out), f64(art.lse)
    assert np.all(np.isfinite(got_l))
    rng = np.random.default_rng(47)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 255, 256, ap.L // 2, ap.L - 1],
                                     rng.integers(0, ap.R, size=6)]))
    heads = [0, ap.n_local - 1, int(rng.integers(1, ap.n_local - 1))]
    latent = _doc_latent(ap)
    out, lse = orc.build_artifact(latent, orc.bf16_to_f64(ap.q[rows]), orc.bf16_to_f64(ap.W), ap.H,
                                  ap.n_local, ap.scale, ap.doc_rows, row_ids=rows, heads=heads)
    ma, r = check_out(got_o[rows][:, heads], out, what="sampled out")
    # rows 0, 1, 63, 64 and 255 see fewer than FEW_KEYS keys (random weights,
    # as in the benchmark's build): their derived bound; the rest the bar
    e = check_lse(got_l[rows][:, heads], lse, tol=_lse_tol(ap, rows, heads, latent, False), what="sampled lse")
    say(f"  {len(rows)} rows x {len(heads)} heads: out max-abs {ma:.2e} rel-L2 {r:.2e}, lse {e:.2e}")
