"""Pins for the fp64 oracle: each test checks the oracle against something
other than itself (brute force, closed forms, identities the pages state,
library routines, page-printed values), chosen so that a dropped term, a
wrong sign, index or operand order fails at least one of them."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
from oracle import mla_oracle as orc

# ---------------------------------------------------------------- number codecs

def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3fn_decode_all_256_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2                       # 0x7F and 0xFF
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    # a few values fixed by the format definition itself
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0


def test_bf16_rne_matches_torch_including_ties():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, size=50000, dtype=np.uint64).astype(np.uint32)
    u[:1000] = (u[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.f32_to_bf16_bits_rne(x)
    assert np.array_equal(ref, got)


def test_fp8_expected_gather_bits_match_torch_arithmetic():
    """bf16(fp32(e4m3) * fp32 scale) computed by torch's own casts and fp32 multiply."""
    prob = mi.make_problem(2, [128, 64], [1, 1], 64, "fp8", seed=11)
    for r in range(2):
        C = int(prob.ctx_len[r])
        got = orc.gather_fp8_expected_bits(prob.pool, prob.block_table, r, 0, C)
        # rebuild with torch from the raw block bytes, token by token
        for t in range(0, C, 7):
            blk = int(prob.block_table[r, t // 64]); s = t % 64
            raw = prob.pool[blk]
            codes = torch.from_numpy(raw[s * 512:(s + 1) * 512].copy()).view(torch.float8_e4m3fn)
            sc = torch.from_numpy(raw[40960 + 4 * s:40960 + 4 * s + 4].copy()).view(torch.float32)
            val = (codes.to(torch.float32) * sc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(val, got[t, :512])
            rope = raw[32768 + s * 128:32768 + (s + 1) * 128].copy().view(np.uint16)
            assert np.array_equal(rope, got[t, 512:])


# ---------------------------------------------------------------- gather

def test_gather_is_block_table_indexing_bruteforce():
    """Payload of pool[b, s, c] encodes (b, s, c); gather of any range must
    return exactly the payloads a per-token walk of the block table names."""
    NB = 9
    pool = np.zeros((NB, 64, 576), dtype=np.uint16)
    for b in range(NB):
        for s in range(64):
            pool[b, s, :] = (b * 64 + s) % 65536
            pool[b, s, 575] = b
    bt = np.array([[5, 2, 7, 0], [8, 1, 3, 6]], dtype=np.int32)
    for req, start, length in [(0, 0, 192), (0, 70, 50), (1, 63, 130), (1, 255, 1), (0, 10, 0)]:
        got = orc.gather_bf16_bits(pool, bt, req, start, length)
        assert got.shape == (length, 576)
        for i in range(length):
            t = start + i
            blk = [int(x) for x in bt[req]][t // 64]
            assert got[i, 0] == blk * 64 + t % 64 and got[i, 575] == blk


def test_fp8_gather_closed_form_values():
    """A hand-built fp8 block: code 0x38 (1.0) with scale 0.5 -> 0.5;
    code 0xC0 (-2.0) with scale 3 -> -6; rope bits copied."""
    pool = np.zeros((2, orc.fp8_block_bytes()), dtype=np.uint8)
    pool[1, 5 * 512:(5 + 1) * 512] = 0x38
    pool[1, 5 * 512 + 7] = 0xC0
    pool[1, 40960 + 4 * 5:40960 + 4 * 6] = np.array([0.5], np.float32).view(np.uint8)
    pool[1, 32768 + 5 * 128:32768 + 5 * 128 + 2] = np.array([0x3F80], np.uint16).view(np.uint8)
    bt = np.array([[1]], dtype=np.int32)
    x = orc.gather_fp8_f64(pool, bt, 0, 5, 1)
    assert x[0, 0] == 0.5 and x[0, 7] == -1.0 and x[0, 512] == 1.0 and x[0, 513] == 0.0
    pool[1, 40960 + 4 * 5:40960 + 4 * 6] = np.array([3.0], np.float32).view(np.uint8)
    x = orc.gather_fp8_f64(pool, bt, 0, 5, 1)
    assert x[0, 7] == -6.0 and x[0, 1] == 3.0


# ---------------------------------------------------------------- attention

def _bruteforce_prefill(prob):
    """Pure-Python loops with math.fsum for every sum: decompression, scores,
    softmax and output. Independent of the oracle's NumPy code."""
    H = prob.H
    W = [[float(v) for v in row] for row in orc.bf16_to_f64(prob.W)]
    cu = prob.cu_ext()
    out = {}
    for r in range(prob.B):
        C, E = int(prob.ctx_len[r]), int(prob.ext_len[r])
        lat = []
        for t in range(C):
            blk = int(prob.block_table[r, t // 64])
            lat.append([float(v) for v in orc.bf16_to_f64(prob.pool[blk, t % 64])])
        for t in range(E):
            lat.append([float(v) for v in orc.bf16_to_f64(prob.ext_latent[cu[r] + t])])
        o_r = np.zeros((E, H, 128)); l_r = np.zeros((E, H))
        for h in range(H):
            kn = [[math.fsum(lat[j][i] * W[i][h * 128 + d] for i in range(512)) for d in range(128)]
                  for j in range(C + E)]
            vv = [[math.fsum(lat[j][i] * W[i][H * 128 + h * 128 + d] for i in range(512)) for d in range(128)]
                  for j in range(C + E)]
            for i in range(E):
                q = [float(x) for x in orc.bf16_to_f64(prob.q[cu[r] + i, h])]
                s = []
                for j in range(C + i + 1):
                    dot = math.fsum([q[d] * kn[j][d] for d in range(128)] +
                                    [q[128 + d] * lat[j][512 + d] for d in range(64)])
                    s.append(prob.scale * dot)
                m = max(s)
                e = [math.exp(x - m) for x in s]
                Z = math.fsum(e)
                l_r[i, h] = m + math.log(Z)
                for d in range(128):
                    o_r[i, h, d] = math.fsum(e[j] * vv[j][d] for j in range(len(s))) / Z
        out[r] = (o_r, l_r)
    return out


def test_attention_matches_bruteforce_loops():
    prob = mi.make_problem(2, [5], [3], 128, "bf16", seed=21)
    # 5 context tokens need one block; the unused slots stay unread
    ref = orc.prefill_reference(prob)
    bf = _bruteforce_prefill(prob)
    o, l = ref[0]
    np.testing.assert_allclose(o, bf[0][0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, bf[0][1], rtol=1e-13, atol=1e-13)


def _selection_W(H, vsel, ksel=None):
    """kv_b_proj whose columns each copy one latent coordinate: W_UV^h[:, d]
    = e_{vsel(h,d)}, W_UK^h[:, d] = e_{ksel(h,d)} (or 0)."""
    W = np.zeros((512, H * 256), dtype=np.float32)
    for h in range(H):
        for d in range(128):
            W[vsel(h, d), H * 128 + h * 128 + d] = 1.0
            if ksel is not None:
                W[ksel(h, d), h * 128 + d] = 1.0
    return mi.f32_to_bf16_bits(W)


def test_zero_query_gives_uniform_average_and_log_count():
    """q = 0: every visible key has weight 1/n, so out = mean of visible v and
    lse = ln n. With a selection kv_b_proj, v_h[:, d] is latent column
    (3h + 5d) % 512, so the expected value is a plain column mean of the
    gathered records. n for extend row i is C + i + 1 (causal, bottom-right)."""
    H = 3
    prob = mi.make_problem(H, [128, 64], [4, 6], 64, "bf16", seed=22, extra_blocks=2)
    vsel = lambda h, d: (3 * h + 5 * d) % 512
    prob.W = _selection_W(H, vsel)
    prob.q[:] = 0
    ref = orc.prefill_reference(prob)
    cu = prob.cu_ext()
    for r in range(prob.B):
        C, E = int(prob.ctx_len[r]), int(prob.ext_len[r])
        recs = [orc.bf16_to_f64(prob.pool[prob.block_table[r, t // 64], t % 64]) for t in range(C)]
        recs += [orc.bf16_to_f64(prob.ext_latent[cu[r] + t]) for t in range(E)]
        recs = np.array(recs)
        for i in range(E):
            n = C + i + 1
            assert ref[r][1][i] == pytest.approx(np.full(H, math.log(n)), abs=1e-12)
            for h in range(H):
                cols = [vsel(h, d) for d in range(128)]
                np.testing.assert_allclose(ref[r][0][i, h], recs[:n, cols].mean(axis=0), atol=1e-12)


def test_single_visible_key_returns_its_value_and_score():
    """With no context, extend row 0 sees only key 0: out = v_0 and lse = s_0.
    q_nope = 0 and q_rope = 2 e_5 give s_0 = scale * 2 * k_rope_0[5]."""
    H = 2
    prob = mi.make_problem(H, [0], [3], 64, "bf16", seed=23)
    vsel = lambda h, d: (7 * h + d) % 512
    prob.W = _selection_W(H, vsel)
    prob.q[:] = 0
    prob.q[0, :, 128 + 5] = mi.f32_to_bf16_bits(np.array([2.0], np.float32))[0]
    ref = orc.prefill_reference(prob)
    lat0 = orc.bf16_to_f64(prob.ext_latent[0])
    for h in range(H):
        np.testing.assert_allclose(ref[0][0][0, h], lat0[[vsel(h, d) for d in range(128)]], atol=1e-13)
        assert ref[0][1][0, h] == pytest.approx(prob.scale * 2.0 * lat0[512 + 5], abs=1e-13)


def test_two_keys_pin_scale_nope_and_rope_terms():
    """Two visible keys: weights are the logistic function of scale*(s0-s1).
    The nope part goes through W_UK (selection of latent coord ksel), the rope
    part through the shared k_rope; both must appear with the 1/sqrt(192)
    scale."""
    H = 2
    ksel = lambda h, d: (11 * h + 3 * d + 1) % 512
    vsel = lambda h, d: (5 * h + d + 100) % 512
    prob = mi.make_problem(H, [0], [2], 64, "bf16", seed=24)
    prob.W = _selection_W(H, vsel, ksel)
    q = np.zeros((2, H, 192), np.float32)
    q[1, 0, 4] = 1.5        # head 0: nope coordinate 4 -> latent coord ksel(0, 4)
    q[1, 1, 128 + 9] = -0.75  # head 1: rope coordinate 9
    prob.q = mi.f32_to_bf16_bits(q)
    ref = orc.prefill_reference(prob)
    lat = orc.bf16_to_f64(prob.ext_latent[:2])
    sc = 1.0 / math.sqrt(192.0)
    for h, s in [(0, [1.5 * lat[j, ksel(0, 4)] for j in range(2)]),
                 (1, [-0.75 * lat[j, 512 + 9] for j in range(2)])]:
        a = sc * s[0]; b = sc * s[1]
        w0 = 1.0 / (1.0 + math.exp(b - a))
        v = lat[:, [vsel(h, d) for d in range(128)]]
        np.testing.assert_allclose(ref[0][0][1, h], w0 * v[0] + (1 - w0) * v[1], atol=1e-12)
        assert ref[0][1][1, h] == pytest.approx(max(a, b) + math.log1p(math.exp(-abs(a - b))), abs=1e-12)


# ---------------------------------------------------------------- merge

def _rand_head(rng, n_q=6, n_k=40):
    q = rng.standard_normal((n_q, 192))
    kn = rng.standard_normal((n_k, 128))
    kr = rng.standard_normal((n_k, 64))
    v = rng.standard_normal((n_k, 128))
    return q, kn, kr, v


def test_merge_identity_every_cut_point():
    """Splitting the keys at any point and merging the two (out, lse) by the
    log-sum-exp rule reproduces the unsplit softmax."""
    rng = np.random.default_rng(3)
    q, kn, kr, v = _rand_head(rng)
    sc = 0.3
    o, l = orc.attend(q, kn, kr, v, sc)
    for cut in range(0, 41):
        oa, la = orc.attend(q, kn[:cut], kr[:cut], v[:cut], sc)
        ob, lb = orc.attend(q, kn[cut:], kr[cut:], v[cut:], sc)
        om, lm = orc.merge_states(oa, la, ob, lb)
        np.testing.assert_allclose(om, o, atol=1e-12)
        np.testing.assert_allclose(lm, l, atol=1e-12)


def test_merge_three_segments_any_order_and_empty_identity():
    rng = np.random.default_rng(4)
    q, kn, kr, v = _rand_head(rng, n_k=30)
    sc = 0.2
    o, l = orc.attend(q, kn, kr, v, sc)
    segs = [(0, 7), (7, 19), (19, 30)]
    parts = [orc.attend(q, kn[a:b], kr[a:b], v[a:b], sc) for a, b in segs]
    for order in [(0, 1, 2), (2, 0, 1), (1, 2, 0)]:
        acc = (np.zeros_like(o), np.full_like(l, -np.inf))
        for i in order:
            acc = orc.merge_states(acc[0], acc[1], *parts[i])
        np.testing.assert_allclose(acc[0], o, atol=1e-12)
        np.testing.assert_allclose(acc[1], l, atol=1e-12)
    # empty segment is the identity; both empty gives (0, -inf) without NaN
    e_o, e_l = np.zeros_like(o), np.full_like(l, -np.inf)
    om, lm = orc.merge_states(o, l, e_o, e_l)
    assert np.array_equal(om, o) and np.array_equal(lm, l)
    om, lm = orc.merge_states(e_o, e_l, e_o, e_l)
    assert np.all(om == 0) and np.all(np.isneginf(lm)) and not np.any(np.isnan(om))


def test_merge_weights_closed_form():
    """lse_a = ln 3, lse_b = ln 1: weights 3/4 and 1/4; merged lse = ln 4."""
    oa = np.full((1, 4), 2.0); ob = np.full((1, 4), -2.0)
    om, lm = orc.merge_states(oa, np.array([math.log(3.0)]), ob, np.array([0.0]))
    np.testing.assert_allclose(om, np.full((1, 4), 1.0), atol=1e-15)
    assert lm[0] == pytest.approx(math.log(4.0), abs=1e-15)


def test_chunked_loop_equals_plain_definition():
    """The chunked context loop plus causal extend and merges equals the
    single-softmax definition for every chunk size, including a ragged last
    chunk and a chunk larger than the context."""
    prob = mi.make_problem(2, [192, 64, 0], [5, 3, 4], 64, "bf16", seed=25, extra_blocks=1)
    ref = orc.prefill_reference(prob)
    for chunk in [1, 50, 64, 100, 1000]:
        got = orc.chunked_prefill_f64(prob, chunk)
        for r in range(prob.B):
            np.testing.assert_allclose(got[r][0], ref[r][0], atol=1e-12)
            np.testing.assert_allclose(got[r][1], ref[r][1], atol=1e-12)


def test_chunked_loop_equals_plain_definition_fp8_cache():
    prob = mi.make_problem(2, [128, 64], [3, 2], 64, "fp8", seed=26)
    ref = orc.prefill_reference(prob)
    got = orc.chunked_prefill_f64(prob, 40)
    for r in range(prob.B):
        np.testing.assert_allclose(got[r][0], ref[r][0], atol=1e-12)
        np.testing.assert_allclose(got[r][1], ref[r][1], atol=1e-12)


def test_absorbed_form_equals_decompressed_form():
    """Folding W_UK into the query and applying W_UV after attention gives
    the same scores and outputs as decompressing per-head keys and values."""
    prob = mi.make_problem(3, [128], [8], 64, "bf16", seed=27)
    W = orc.bf16_to_f64(prob.W)
    lat = orc.request_keys_f64(prob, 0)
    vis = orc.causal_visible(8, 128)
    for h in range(3):
        q = orc.bf16_to_f64(prob.q[:, h])
        kn, v = orc.decompress_head(lat[:, :512], W, 3, h)
        o1, l1 = orc.attend(q, kn, lat[:, 512:], v, prob.scale, vis)
        o2, l2 = orc.attend_absorbed(q, lat, W, 3, h, prob.scale, vis)
        np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- rope

def _rot_complex(x, pos, base=10000.0):
    """Reference rotation by complex multiplication (interleaved pairs)."""
    z = x[..., 0::2] + 1j * x[..., 1::2]
    k = np.arange(32)
    z = z * np.exp(1j * pos * base ** (-2.0 * k / 64.0))
    y = np.empty_like(x)
    y[..., 0::2], y[..., 1::2] = z.real, z.imag
    return y


@pytest.mark.parametrize("delta", [0, 1, 4096, 2 ** 18])
def test_rope_relocation_identity(delta):
    """q at request position delta+L+i rotated by -delta, dotted with a
    canonical key at position j, equals the unrotated dot under the relative
    rotation j-(L+i), and equals direct placement of the key at delta+j."""
    rng = np.random.default_rng(5)
    L, i = 300, 7
    q0 = rng.standard_normal(64); k0 = rng.standard_normal((20, 64))
    j = np.arange(20) * 13
    q = _rot_complex(q0, delta + L + i)
    kc = _rot_complex(k0, j[:, None])
    lhs = kc @ orc.relocate_q(q, delta)
    direct = orc.rope_rotate(kc, float(delta)) @ q
    rel = np.array([_rot_complex(k0[t], j[t] - (L + i)) @ q0 for t in range(20)])
    np.testing.assert_allclose(lhs, rel, atol=1e-9)
    np.testing.assert_allclose(direct, rel, atol=1e-9)


def test_rope_matches_complex_rotation_and_group_laws():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 64))
    for p in [0.0, 1.0, -3.0, 4096.0, 262144.0]:
        np.testing.assert_allclose(orc.rope_rotate(x, p), _rot_complex(x, p), atol=1e-9)
    a, b = 17.0, 4096.0
    np.testing.assert_allclose(orc.rope_rotate(orc.rope_rotate(x, a), b), orc.rope_rotate(x, a + b), atol=1e-9)
    np.testing.assert_allclose(orc.rope_rotate(orc.rope_rotate(x, a), -a), x, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(orc.rope_rotate(x, b), axis=1), np.linalg.norm(x, axis=1))
    # half-split pairing is the interleaved rotation under the pair permutation
    perm = np.empty(64, dtype=int); perm[0::2] = np.arange(32); perm[1::2] = np.arange(32, 64)
    np.testing.assert_allclose(orc.rope_rotate(x[:, perm], a, pairing="interleaved"),
                               orc.rope_rotate(x, a, pairing="half")[:, perm], atol=1e-12)


# ---------------------------------------------------------------- equation 4

def test_equation4_exact_under_full_recompute():
    """With the artifact equal to the true Local-head outputs, sliced
    projection plus shared W_b equals attention over all heads followed by
    one unsliced [O_L | O_G] [W_aL ; W_aG] W_b."""
    prob = mi.make_reuse_problem(H=4, n_local=3, L=192, T=10, delta=4096, P=3,
                                 d_mid=16, d_model=24, chunk=64, seed=31)
    ref = orc.reuse_reference(prob)
    # true Local outputs for every row (full recomputation)
    full = orc.reuse_reference(prob, global_rows=None)
    prob_all = mi.make_reuse_problem(H=4, n_local=3, L=192, T=10, delta=4096, P=10,
                                     d_mid=16, d_model=24, chunk=64, seed=31)
    # P = T protects every row: recomputed Local outputs for all rows
    allrows = orc.reuse_reference(prob_all)
    O_L = allrows["rec"]                      # [T, 3, 128] since prot = 0..T-1
    assert np.array_equal(prob_all.prot_rows, np.arange(10))
    WaL, WaG, Wb = (orc.bf16_to_f64(x) for x in (prob_all.WaL, prob_all.WaG, prob_all.Wb))
    y = orc.head_partition_merge(O_L, allrows["O_G"], WaL, WaG, Wb)
    O_all = np.concatenate([O_L, allrows["O_G"]], axis=1).reshape(10, -1)
    y2 = O_all @ np.concatenate([WaL, WaG], axis=0) @ Wb
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(allrows["y"], y2, rtol=1e-12, atol=1e-12)
    assert full["y"].shape == ref["y"].shape == (10, 24)


def test_protected_rows_replace_not_add():
    """Protected rows take the recomputed value; unprotected rows keep the
    artifact; with rec equal to the artifact's own rows nothing changes."""
    rng = np.random.default_rng(7)
    art = rng.standard_normal((12, 3, 128)); rec = rng.standard_normal((4, 3, 128))
    prot = np.array([1, 4, 5, 11])
    o = orc.replace_protected(art, rec, prot)
    assert np.array_equal(o[prot], rec)
    keep = np.setdiff1d(np.arange(12), prot)
    assert np.array_equal(o[keep], art[keep])
    assert np.array_equal(orc.replace_protected(art, art[prot], prot), art)


def test_reuse_reference_against_relocated_query_bruteforce():
    """Config-5 style reference (direct placement of keys at delta+j) against
    a loop that relocates the queries by -delta with complex rotations and
    attends to canonical keys."""
    prob = mi.make_reuse_problem(H=3, n_local=2, L=128, T=6, delta=4096, P=2,
                                 d_mid=8, d_model=8, chunk=64, seed=32)
    ref = orc.reuse_reference(prob)
    W = orc.bf16_to_f64(prob.W)
    lat = np.array([orc.bf16_to_f64(prob.pool[prob.block_table[0, t // 64], t % 64]) for t in range(128)])
    q = orc.bf16_to_f64(prob.q)
    def attend_loop(qv):
        qv = qv.copy()
        z = qv[128:][0::2] + 1j * qv[128:][1::2]
        z = z * np.exp(-1j * prob.delta * 10000.0 ** (-2.0 * np.arange(32) / 64.0))
        qv[128:][0::2], qv[128:][1::2] = z.real, z.imag
        return qv
    for h, rows, got_o, got_l in [(2, range(6), ref["O_G"][:, 0], ref["lse_G"][:, 0])] + \
            [(h, prob.prot_rows, ref["rec"][:, h], ref["rec_lse"][:, h]) for h in range(2)]:
        kn = lat[:, :512] @ W[:, h * 128:(h + 1) * 128]
        v = lat[:, :512] @ W[:, 3 * 128 + h * 128:3 * 128 + (h + 1) * 128]
        for gi, i in enumerate(rows):
            qv = attend_loop(q[i, h])
            s = np.array([math.fsum(list(qv[:128] * kn[j]) + list(qv[128:] * lat[j, 512:]))
                          for j in range(128)]) * prob.scale
            m = s.max(); e = np.exp(s - m); Z = math.fsum(e)
            np.testing.assert_allclose(got_o[gi], (e @ v) / Z, atol=1e-9)
            assert got_l[gi] == pytest.approx(m + math.log(Z), abs=1e-9)


# ---------------------------------------------------------------- layout

def _read_golden(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        rows.append(line.split())
    return rows


def test_latent_record_layout_and_kv_size_table():
    """576 elements (1152 B bf16) per token per layer; exact MHA/MLA byte ratio
    65536/1152 = 56.89. The MHA column of the page's KV-size table is exact
    in GiB for 61 layers; the printed MLA columns and ratios are rounded
    (about 1.2 percent high) and are checked only to 1.5 percent."""
    assert orc.latent_record_elems() == 576
    assert orc.latent_record_elems() * 2 == 1152
    mha = orc.mha_bytes_per_token_layer(128, 128)
    assert mha == 65536
    assert mha / 1152 == pytest.approx(56.8889, abs=1e-4)
    assert orc.fp8_block_bytes() == 41216 == mi.FP8_BLOCK_BYTES
    for ctx, mha_p, unit, mla_p, fp8_p, ratio_p in _read_golden("kv_cache_table_dsv3.txt"):
        tokens = int(ctx)
        gib = 1024 ** 3 if unit == "GB" else 1000 * 1024 ** 3
        mha_exact = tokens * 61 * mha / gib
        assert mha_exact == pytest.approx(float(mha_p), abs=0.051)
        mla_exact_gib = tokens * 61 * 1152 / 1024 ** 3
        assert float(mla_p) == pytest.approx(mla_exact_gib, rel=0.015)
        assert float(ratio_p) == pytest.approx(65536 / 1152, rel=0.015)


# ---------------------------------------------------------------- cache write path (fp8 encode)

def _e4m3_finite_values():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    return codes, orc.e4m3fn_to_f64(codes)


def test_e4m3_encode_matches_torch_cast_on_ties_and_neighbours():
    """Every midpoint between adjacent E4M3FN values (the round-to-even ties),
    one fp32 ulp either side of it, every value itself and random values,
    against torch's float8_e4m3fn cast (a library routine)."""
    _, vals = _e4m3_finite_values()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[:-1] + pos[1:]) / 2.0
    x = np.concatenate([pos, mids]).astype(np.float32)
    x = np.concatenate([x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))])
    rng = np.random.default_rng(90)
    x = np.concatenate([x, (rng.standard_normal(20000) * 40).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-3).astype(np.float32)])
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    x = np.concatenate([x, -x])
    got = orc.e4m3fn_encode_rne(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_encode_decode_round_trip_every_code():
    codes, vals = _e4m3_finite_values()
    assert np.array_equal(orc.e4m3fn_encode_rne(vals.astype(np.float32)), codes)


def test_quantize_token_closed_form_record():
    """c_kv = (1, -2, 0.5, 0, ...): max |x| = 2, scale = fp32(2/448); x/scale
    = 224, -448, 112 -> codes 0x76 (1.75 * 2^7), 0xFE (-1.75 * 2^8), 0x6E
    (1.75 * 2^6), zeros -> 0x00. An all-zero record gets scale 0 and zero
    codes."""
    rec = np.zeros((2, 512), dtype=np.float32)
    rec[0, :3] = [1.0, -2.0, 0.5]
    bits = (rec.view(np.uint32) >> 16).astype(np.uint16)
    codes, scale = orc.quantize_token_e4m3(bits)
    assert scale[0] == np.float32(2.0) / np.float32(448.0) and scale[1] == 0
    assert list(codes[0, :4]) == [0x76, 0xFE, 0x6E, 0x00] and not codes[0, 4:].any()
    assert not codes[1].any()


def test_quantize_token_matches_the_generator_quantiser():
    """The generator's own quantiser (torch's cast) on random records, plus
    records whose maximum sits at a tie: identical codes and scales."""
    rng = np.random.default_rng(91)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[5] = 0.0
    x[6, 7] = 9.0
    bits = mi.f32_to_bf16_bits(x)
    c1, s1 = orc.quantize_token_e4m3(bits)
    c2, s2 = mi.quantize_rows_e4m3(bits)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(c1, c2)
    # the largest magnitude of a nonzero record maps to +-448 exactly
    amax_code = c1[np.arange(64), np.argmax(np.abs(orc.bf16_to_f64(bits)), axis=1)]
    assert np.all((amax_code[np.arange(64) != 5] & 0x7F) == 0x7E)


def test_cache_append_expected_places_records_and_touches_nothing_else():
    """Hand-built pools: request 0 appends 3 tokens at position 62 (crossing
    into its second block), request 1 one token at position 0. Each record
    lands in block_table[r][t // 64], slot t % 64, the gather of the written
    range returns it, and every other byte keeps its value."""
    rng = np.random.default_rng(92)
    bt = np.array([[3, 1], [0, 2]], dtype=np.int32)
    new = mi.f32_to_bf16_bits(rng.standard_normal((4, 576)).astype(np.float32))
    pos0, lens = [62, 0], [3, 1]
    pool = np.full((4, 64, 576), 0x7FC0, dtype=np.uint16)
    out = orc.cache_append_expected(pool, bt, pos0, lens, new, "bf16")
    assert np.array_equal(out[3, 62], new[0]) and np.array_equal(out[3, 63], new[1])
    assert np.array_equal(out[1, 0], new[2]) and np.array_equal(out[0, 0], new[3])
    assert np.array_equal(orc.gather_bf16_bits(out, bt, 0, 62, 3), new[:3])
    changed = np.any(out != pool, axis=-1)
    assert changed.sum() == 4
    fp = np.full((4, orc.fp8_block_bytes()), 0xA5, dtype=np.uint8)
    out8 = orc.cache_append_expected(fp, bt, pos0, lens, new, "fp8")
    codes, scale = orc.quantize_token_e4m3(new[:, :512])
    back = orc.gather_fp8_f64(out8, bt, 0, 62, 3)
    assert np.array_equal(back[:, :512], orc.e4m3fn_to_f64(codes[:3]) * scale[:3, None].astype(np.float64))
    assert np.array_equal(back[:, 512:], orc.bf16_to_f64(new[:3, 512:]))
    # bytes of blocks/slots not written are untouched
    written = np.zeros_like(fp, dtype=bool)
    for b, sl in [(3, 62), (3, 63), (1, 0), (0, 0)]:
        written[b, sl * 512:(sl + 1) * 512] = True
        written[b, 32768 + sl * 128:32768 + (sl + 1) * 128] = True
        written[b, 40960 + sl * 4:40960 + (sl + 1) * 4] = True
    assert np.all(out8[~written] == 0xA5)


# ---------------------------------------------------------------- multi-document (segmented) reuse

def test_segmented_runtime_form_equals_direct_placement():
    """Per-document relocation + canonical attention + LSE merge (the runtime
    form) equals one softmax over all documents' keys at their request
    positions (the definition), for Global and protected Local rows."""
    prob = mi.make_multidoc_problem(H=4, n_local=3, doc_lens=(128, 64, 192), T=12, P=3, seed=93,
                                    d_mid=128, d_model=128)
    ref = orc.reuse_reference(prob)
    rows = np.arange(prob.T)
    o, l = orc.segmented_attention(prob, 3, rows)
    assert np.allclose(o, ref["O_G"][:, 0], rtol=1e-10, atol=1e-12)
    assert np.allclose(l, ref["lse_G"][:, 0], rtol=0, atol=1e-10)
    prot = np.asarray(prob.prot_rows)
    for h in range(3):
        o, l = orc.segmented_attention(prob, h, prot)
        assert np.allclose(o, ref["rec"][:, h], rtol=1e-10, atol=1e-12)
        assert np.allclose(l, ref["rec_lse"][:, h], rtol=0, atol=1e-10)


def test_each_document_uses_its_own_offset():
    """A stored k_rope is the key rotated at its canonical position inside its
    own document, so each document must be placed by its own delta_d: moving
    one document by one position, or placing every document at the first
    one's offset, changes the result far beyond the parity tolerance."""
    prob = mi.make_multidoc_problem(H=4, n_local=3, doc_lens=(64, 128, 64), T=10, P=2, seed=94,
                                    d_mid=128, d_model=128)
    base = orc.reuse_reference(prob)["O_G"]
    docs = [dict(d) for d in prob.documents()]
    docs[1]["delta"] += 1
    moved = orc.reuse_reference(dataclasses.replace(prob, docs=docs))["O_G"]
    same = [dict(d, delta=prob.documents()[0]["delta"]) for d in prob.documents()]
    flat = orc.reuse_reference(dataclasses.replace(prob, docs=same))["O_G"]
    for other in (moved, flat):
        assert np.linalg.norm(other - base) / np.linalg.norm(base) > 0.02


# ---------------------------------------------------------------- offline artifact (MLA-Off)

def test_fnv1a64_published_vectors_and_token_framing():
    """FNV-1a 64 against the published test vectors of its authors, and the
    token framing: each id as 4 little-endian bytes."""
    assert orc.fnv1a64(b"") == 0xcbf29ce484222325
    assert orc.fnv1a64(b"a") == 0xaf63dc4c8601ec8c
    assert orc.fnv1a64(b"foobar") == 0x85944171f73967e8
    assert orc.token_bytes([0x64636261, -1, 7]) == b"abcd" + b"\xff" * 4 + b"\x07\x00\x00\x00"
    assert orc.artifact_token_hash([]) == 0xcbf29ce484222325
    # order matters, and a single changed id changes the hash
    assert orc.artifact_token_hash([1, 2]) != orc.artifact_token_hash([2, 1])
    assert orc.artifact_token_hash([5, 9, 11]) != orc.artifact_token_hash([5, 9, 12])


def _meta(**kw):
    m = dict(generation=3, token_hash=0x1234, n_tokens=1088, n_heads=64, n_local=56, d_c=512, d_rope=64,
             d_nope=128, d_v=128, rope_base=10000.0, n_layers=37, layer_mask=(1 << 37) - 1)
    m.update(kw)
    return m


def test_artifact_check_reasons_and_their_order():
    """Each single mismatch gives its own reason; with several, the first in
    the page's list (layers, tokens, profile, generation) wins; a request
    that needs fewer layers than the artifact holds is valid."""
    a = _meta()
    assert orc.artifact_check_reason(a, _meta()) == 0
    assert orc.artifact_check_reason(a, _meta(layer_mask=1 << 3)) == 0
    assert orc.artifact_check_reason(_meta(layer_mask=a["layer_mask"] & ~(1 << 20)), _meta()) == 1
    assert orc.artifact_check_reason(a, _meta(token_hash=0x1235)) == 2
    assert orc.artifact_check_reason(a, _meta(n_tokens=1089)) == 2
    for f, v in [("n_heads", 128), ("n_local", 48), ("d_c", 256), ("d_rope", 32), ("d_nope", 64),
                 ("d_v", 64), ("rope_base", 50000.0), ("n_layers", 55)]:
        assert orc.artifact_check_reason(a, _meta(**{f: v})) == 3, f
    assert orc.artifact_check_reason(a, _meta(generation=4)) == 4
    assert orc.artifact_check_reason(a, _meta(generation=2)) == 4
    assert orc.artifact_check_reason(_meta(layer_mask=0), _meta(token_hash=1, n_heads=1, generation=9)) == 1
    assert orc.artifact_check_reason(a, _meta(token_hash=1, n_heads=1, generation=9)) == 2
    assert orc.artifact_check_reason(a, _meta(n_heads=1, generation=9)) == 3


def _art_inputs(prob):
    lat = np.array([orc.bf16_to_f64(prob.pool[prob.block_table[0, t // 64], t % 64]) for t in range(prob.L)])
    return lat, orc.bf16_to_f64(prob.q), orc.bf16_to_f64(prob.W)


def test_artifact_first_document_row_sees_one_key():
    """Document row 0 sees only key 0: out = v_0 (its W_UV product) and
    lse = its one score, s_0 = scale (q_nope . c W_UK + q_rope . k_rope)."""
    prob = mi.make_artifact_problem(H=3, n_local=2, L=70, extra_rows=2, seed=41)
    lat, q, W = _art_inputs(prob)
    out, lse = orc.build_artifact(lat, q, W, 3, 2, prob.scale, doc_rows=True)
    for h in range(2):
        k = lat[0, :512] @ W[:, h * 128:(h + 1) * 128]
        v = lat[0, :512] @ W[:, 3 * 128 + h * 128:3 * 128 + (h + 1) * 128]
        s0 = prob.scale * (q[0, h, :128] @ k + q[0, h, 128:] @ lat[0, 512:])
        np.testing.assert_allclose(out[0, h], v, rtol=1e-12, atol=1e-14)
        assert lse[0, h] == pytest.approx(s0, abs=1e-12)


def test_artifact_bruteforce_loops():
    """Every row and Local head of a tiny artifact against per-element fsum
    loops: document row t over keys 0..t, rows after the document over every
    key; heads >= n_local are not part of the artifact."""
    prob = mi.make_artifact_problem(H=3, n_local=2, L=9, extra_rows=3, seed=42)
    lat, q, W = _art_inputs(prob)
    out, lse = orc.build_artifact(lat, q, W, 3, 2, prob.scale, doc_rows=True)
    assert out.shape == (12, 2, 128) and lse.shape == (12, 2)
    for h in range(2):
        K = [[math.fsum(lat[t, c] * W[c, h * 128 + d] for c in range(512)) for d in range(128)] for t in range(9)]
        V = [[math.fsum(lat[t, c] * W[c, 3 * 128 + h * 128 + d] for c in range(512)) for d in range(128)]
             for t in range(9)]
        for r in range(12):
            keys = range(r + 1) if r < 9 else range(9)
            s = [prob.scale * math.fsum([q[r, h, d] * K[t][d] for d in range(128)] +
                                        [q[r, h, 128 + j] * lat[t, 512 + j] for j in range(64)]) for t in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            Z = math.fsum(e)
            o = [math.fsum(e[i] * V[t][d] for i, t in enumerate(keys)) / Z for d in range(128)]
            np.testing.assert_allclose(out[r, h], o, rtol=1e-10, atol=1e-12)
            assert lse[r, h] == pytest.approx(m + math.log(Z), abs=1e-10)
    # rows after the document alone (doc_rows=False) are the same rows
    out2, lse2 = orc.build_artifact(lat, q[9:], W, 3, 2, prob.scale, doc_rows=False)
    np.testing.assert_allclose(out2, out[9:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse[9:], rtol=0, atol=1e-12)
    # selected rows (a document row and a row after it) and one head
    out3, lse3 = orc.build_artifact(lat, q[[2, 10]], W, 3, 2, prob.scale, doc_rows=True, row_ids=[2, 10],
                                    heads=[1])
    np.testing.assert_allclose(out3[:, 0], out[[2, 10], 1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse3[:, 0], lse[[2, 10], 1], rtol=0, atol=1e-12)


def test_artifact_for_request_rows_equals_their_full_recompute():
    """Built at canonical position zero with the request rows' queries moved
    into the canonical frame, the artifact of rows after the document is the
    Local heads' full recomputation in the request (keys placed at +delta),
    so Equation 4 with it and no protected row gives the full-recompute y."""
    prob = mi.make_reuse_problem(H=4, n_local=3, L=192, T=10, delta=4096, P=10,
                                 d_mid=16, d_model=24, chunk=64, seed=43)
    full = orc.reuse_reference(prob)            # P = T: every Local row recomputed
    lat = np.array([orc.bf16_to_f64(prob.pool[prob.block_table[0, t // 64], t % 64]) for t in range(192)])
    q = orc.bf16_to_f64(prob.q)
    qc = q.copy()
    qc[..., 128:] = orc.relocate_q(q[..., 128:], prob.delta, prob.rope_base)
    out, lse = orc.build_artifact(lat, qc, orc.bf16_to_f64(prob.W), 4, 3, prob.scale, doc_rows=False)
    np.testing.assert_allclose(out, full["rec"], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(lse, full["rec_lse"], rtol=0, atol=1e-9)
    O_L = orc.replace_protected(out, out[:0], np.zeros(0, dtype=np.int64))
    WaL, WaG, Wb = (orc.bf16_to_f64(x) for x in (prob.WaL, prob.WaG, prob.Wb))
    y = orc.head_partition_merge(O_L, full["O_G"], WaL, WaG, Wb)
    np.testing.assert_allclose(y, full["y"], rtol=1e-9, atol=1e-12)


def test_fp8_raw_gather_is_the_stored_record():
    """The raw fp8 gather's three parts are the bytes the block layout puts
    at each token: decoding the codes times the scale gives the dequantised
    c_kv of gather_fp8_f64 exactly, and the rope bits are the same; by brute
    force over the byte offsets of reading R16."""
    import mla_inputs as mi
    prob = mi.make_problem(2, [192, 64 * 5], [1, 1], 128, "fp8", seed=13, extra_blocks=2)
    for r, (s0, n) in enumerate([(5, 150), (64, 256)]):
        codes, rope, sc = orc.gather_fp8_raw(prob.pool, prob.block_table, r, s0, n)
        x = orc.gather_fp8_f64(prob.pool, prob.block_table, r, s0, n)
        assert np.array_equal(orc.e4m3fn_to_f64(codes) * sc.astype(np.float64)[:, None], x[:, :512])
        assert np.array_equal(orc.bf16_to_f64(rope), x[:, 512:])
        for i in (0, n // 2, n - 1):
            t = s0 + i
            blk = prob.block_table[r, t // 64]
            base = prob.pool[blk]
            slot = t % 64
            assert np.array_equal(codes[i], base[slot * 512:(slot + 1) * 512])
            assert rope[i].tobytes() == base[32768 + slot * 128:32768 + (slot + 1) * 128].tobytes()
            assert sc[i].tobytes() == base[40960 + slot * 4:40960 + slot * 4 + 4].tobytes()
