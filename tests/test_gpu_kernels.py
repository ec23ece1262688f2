"""Per-kernel parity on the GPU through the C ABI against the fp64 oracle:
gather (bit-exact), merge, RoPE relocation, decompression, attention and the
head-partition projection, on seeded inputs spanning several tiles plus
ragged tails and the degenerate cases (empty key sets, empty requests)."""
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_long_context_amd as mla
from mla_long_context_amd import prefill as pf
from oracle import mla_oracle as orc

from gpu_util import (GAMMA_512, LSE_ABS, U_BF16, bf16_dev, bits, check_lse, check_out, f64, rel_l2,
                      require_gpu, say)

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")


# ---------------------------------------------------------------- gather

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_gather_bit_exact(dtype):
    require_gpu()
    say(f"gather {dtype}")
    prob = mi.make_problem(4, [256, 64 * 7, 0, 128], [1, 1, 1, 1], 128, dtype, seed=41,
                           extra_blocks=5, poison=True)
    pool = pf.upload_pool(prob, "cuda")
    bt = _i32(prob.block_table)
    # ragged windows: unaligned starts, a zero-length request, block-crossing ranges
    starts = np.array([3, 70, 0, 64]); lens = np.array([250, 301, 0, 64])
    cu = np.concatenate([[0], np.cumsum(lens)])
    out = torch.full((int(cu[-1]) + 1, 576), -7.0, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mla.mla_gather_context(pool, mla.DTYPE_BF16 if dtype == "bf16" else mla.DTYPE_FP8_E4M3,
                           prob.num_blocks, bt, bt.shape[1], _i32(starts), _i32(lens), _i32(cu), 4,
                           int(lens.max()), out, status)
    torch.cuda.synchronize()
    got = bits(out)
    for r in range(4):
        if dtype == "bf16":
            ref = orc.gather_bf16_bits(prob.pool, prob.block_table, r, int(starts[r]), int(lens[r]))
        else:
            ref = orc.gather_fp8_expected_bits(prob.pool, prob.block_table, r, int(starts[r]), int(lens[r]))
        assert np.array_equal(got[cu[r]:cu[r + 1]], ref), f"request {r}"
    # the row after the last request is untouched
    assert np.all(f64(out[-1]) == -7.0)
    assert int(status.item()) == 0
    # no NaN from the poisoned unused blocks leaked
    assert not np.any(np.isnan(f64(out[:-1])))


def test_gather_fp8_every_code():
    """Every E4M3FN code (subnormals, both zeros, +-448 and the two NaN codes)
    in every byte position of a record, under several scales, dequantised
    bit for bit as the oracle's bf16_rne(fp32_rne(decode(code) * scale))."""
    require_gpu()
    rng = np.random.default_rng(43)
    nb = 2
    pool = np.zeros((nb, orc.fp8_block_bytes()), dtype=np.uint8)
    codes = np.zeros((nb, 64, 512), dtype=np.uint8)
    for blk in range(nb):
        for slot in range(64):
            codes[blk, slot] = np.roll(np.tile(np.arange(256, dtype=np.uint8), 2), 7 * slot + 3 * blk)
    pool[:, :mi.FP8_ROPE_OFF] = codes.reshape(nb, -1)
    pool[:, mi.FP8_ROPE_OFF:mi.FP8_SCALE_OFF] = np.frombuffer(
        mi.f32_to_bf16_bits(rng.standard_normal((nb, 64, 64)).astype(np.float32)).tobytes(),
        dtype=np.uint8).reshape(nb, -1)
    scales = np.array([1.0, 1 / 448, 0.37, 2.5e-3, 7.0, 1e-6, 3.3e4, 0.0] * 16, dtype=np.float32).reshape(nb, 64)
    pool[:, mi.FP8_SCALE_OFF:] = scales.view(np.uint8).reshape(nb, -1)
    bt = np.array([[1, 0]], dtype=np.int32)
    out = torch.empty((128, 576), dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mla.mla_gather_context(torch.from_numpy(pool).cuda(), mla.DTYPE_FP8_E4M3, nb, _i32(bt), 2, _i32([0]), _i32([128]),
                           _i32([0, 128]), 1, 128, out, status)
    torch.cuda.synchronize()
    ref = orc.gather_fp8_expected_bits(pool, bt, 0, 0, 128)
    got = bits(out)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} differing elements, first {bad[:4].tolist()}"
    assert int(status.item()) == 0


def test_gather_out_of_range_block_sets_status_and_writes_zeros():
    require_gpu()
    prob = mi.make_problem(1, [128], [1], 64, "bf16", seed=42)
    pool = pf.upload_pool(prob, "cuda")
    bt = prob.block_table.copy()
    bt[0, 1] = prob.num_blocks + 3          # second block points outside the pool
    out = torch.full((128, 576), 5.0, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mla.mla_gather_context(pool, mla.DTYPE_BF16, prob.num_blocks, _i32(bt), bt.shape[1], _i32([0]),
                           _i32([128]), _i32([0, 128]), 1, 128, out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == mla._lib.MLA_ERR_OUT_OF_RANGE
    got = bits(out)
    assert np.array_equal(got[:64], orc.gather_bf16_bits(prob.pool, prob.block_table, 0, 0, 64))
    assert np.all(got[64:] == 0)


# ---------------------------------------------------------------- cache append

def _append_case(dtype, seed):
    """Four requests append ragged runs of new records into a shuffled pool:
    an unaligned start crossing two block boundaries, a run ending exactly at
    a block end, an empty request and a single token. Unused blocks are
    poisoned; the result must equal the oracle's pool byte for byte."""
    rng = np.random.default_rng(seed)
    nb_req = [4, 2, 1, 3]
    NB = sum(nb_req) + 3
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((4, 5), -1, dtype=np.int32)
    k = 0
    for r, n in enumerate(nb_req):
        bt[r, :n] = perm[k:k + n]; k += n
    pos0 = np.array([61, 64, 5, 130], dtype=np.int32)
    lens = np.array([133, 64, 0, 1], dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    new = mi.f32_to_bf16_bits(rng.standard_normal((int(cu[-1]) + 2, 576)).astype(np.float32) * 3)
    new[7, :512] = 0                      # a record of zeros: scale 0
    new[9, 100] = mi.f32_to_bf16_bits(np.array([1e-30], np.float32))[0]   # tiny value next to normal ones
    if dtype == "bf16":
        pool = np.full((NB, 64, 576), 0x7FC0, dtype=np.uint16)
        dpool = bf16_dev(pool)
        cdt = mla.DTYPE_BF16
    else:
        pool = np.full((NB, orc.fp8_block_bytes()), 0xA5, dtype=np.uint8)
        dpool = torch.from_numpy(pool.copy()).to("cuda")
        cdt = mla.DTYPE_FP8_E4M3
    return rng, bt, pos0, lens, cu, new, pool, dpool, cdt, NB


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_cache_append_bit_exact(dtype):
    require_gpu()
    say(f"cache append {dtype}")
    rng, bt, pos0, lens, cu, new, pool, dpool, cdt, NB = _append_case(dtype, 80)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mla.mla_cache_append(dpool, cdt, NB, _i32(bt), bt.shape[1], _i32(pos0), _i32(cu), 4, int(lens.max()),
                         bf16_dev(new), 576, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = orc.cache_append_expected(pool, bt, pos0, lens, new, dtype)
    got = bits(dpool) if dtype == "bf16" else dpool.cpu().numpy()
    assert np.array_equal(got, ref)
    # the gather reads back exactly what the oracle stored (fp8: dequantised)
    out = torch.empty((int(lens[0]), 576), dtype=torch.bfloat16, device="cuda")
    mla.mla_gather_context(dpool, cdt, NB, _i32(bt), bt.shape[1], _i32([pos0[0]]), _i32([lens[0]]),
                           _i32([0, lens[0]]), 1, int(lens[0]), out, status)
    torch.cuda.synchronize()
    if dtype == "bf16":
        assert np.array_equal(bits(out), new[:lens[0]])
    else:
        assert np.array_equal(bits(out), orc.gather_fp8_expected_bits(ref, bt, 0, int(pos0[0]), int(lens[0])))


def test_cache_append_out_of_range_is_reported_and_skipped():
    require_gpu()
    rng, bt, pos0, lens, cu, new, pool, dpool, cdt, NB = _append_case("fp8", 81)
    bt[0, 2] = NB + 5                     # positions 128..191 of request 0 -> invalid block id
    pos_bad = pos0.copy(); pos_bad[3] = 5 * 64 - 1 + 1   # request 3 runs past its block-table row
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mla.mla_cache_append(dpool, cdt, NB, _i32(bt), bt.shape[1], _i32(pos_bad), _i32(cu), 4,
                         int(lens.max()), bf16_dev(new), 576, status)
    torch.cuda.synchronize()
    assert int(status.item()) == mla._lib.MLA_ERR_OUT_OF_RANGE
    # valid positions are written as usual; the skipped ones leave the pool
    # as it was: request 0 keeps positions 61..127 and 192..193, request 1 is
    # whole, request 3 is skipped
    ref = orc.cache_append_expected(pool, bt[0:1], [61], [67], new[0:67], "fp8")
    ref = orc.cache_append_expected(ref, bt[0:1], [192], [2], new[131:133], "fp8")
    ref = orc.cache_append_expected(ref, bt[1:2], [pos0[1]], [lens[1]], new[cu[1]:cu[2]], "fp8")
    assert np.array_equal(dpool.cpu().numpy(), ref)


# ---------------------------------------------------------------- merge

@pytest.mark.parametrize("da,db,do", [(2, 0, 2), (2, 0, 0), (0, 0, 0), (2, 2, 2)])
def test_merge_states(da, db, do):
    require_gpu()
    rng = np.random.default_rng(43)
    rows = 4099
    oa = rng.standard_normal((rows, 128)).astype(np.float32)
    ob = rng.standard_normal((rows, 128)).astype(np.float32)
    la = (rng.standard_normal(rows) * 3 + 8).astype(np.float32)
    lb = (rng.standard_normal(rows) * 3 + 8).astype(np.float32)
    la[:7] = -np.inf; lb[3:11] = -np.inf            # one side empty, and both empty (rows 3..6)
    la[20] = 80.0; lb[20] = -80.0                   # extreme weights
    tdt = {0: torch.bfloat16, 2: torch.float32}
    ta = torch.tensor(oa).to(tdt[da]).cuda(); tb = torch.tensor(ob).to(tdt[db]).cuda()
    tla = torch.tensor(la).cuda(); tlb = torch.tensor(lb).cuda()
    out = torch.empty((rows, 128), dtype=tdt[do], device="cuda")
    lout = torch.empty(rows, dtype=torch.float32, device="cuda")
    mla.mla_merge_states(ta, da, tla, tb, db, tlb, rows, out, do, lout)
    # in place into a, as the chunk loop does
    ta2 = ta.clone(); tla2 = tla.clone()
    mla.mla_merge_states(ta2, da, tla2, tb, db, tlb, rows, ta2, da, tla2)
    torch.cuda.synchronize()
    ref_o, ref_l = orc.merge_states(f64(ta), la.astype(np.float64), f64(tb), lb.astype(np.float64))
    tol = 1e-6 if do == 2 else 2 ** -8
    got = f64(out)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref_o) / np.maximum(np.abs(ref_o), 1.0)) <= tol
    check_lse(f64(lout), ref_l, tol=1e-5)
    if da == do:
        assert torch.equal(ta2, out) and torch.equal(tla2, lout)


@pytest.mark.parametrize("pieces,di,do", [(1, 2, 0), (2, 2, 2), (5, 2, 0), (9, 0, 2), (64, 2, 0)])
def test_merge_states_n(pieces, di, do):
    """mla_merge_states_n against the oracle's pairwise merge folded over the
    pieces: empty pieces, rows with every piece empty, extreme weights, a
    ragged piece count; in place into piece 0 as well."""
    require_gpu()
    rng = np.random.default_rng(45 + pieces)
    rows = 1031
    o = rng.standard_normal((pieces, rows, 128)).astype(np.float32)
    lse = (rng.standard_normal((pieces, rows)) * 3 + 8).astype(np.float32)
    lse[:, :5] = -np.inf                             # every piece empty
    lse[0, 5:40] = -np.inf                           # some pieces empty
    if pieces > 2:
        lse[1:3, 40:60] = -np.inf
    lse[0, 60] = 80.0; lse[-1, 60] = -80.0           # extreme weights
    tdt = {0: torch.bfloat16, 2: torch.float32}
    to = torch.tensor(o).to(tdt[di]).cuda()
    tl = torch.tensor(lse).cuda()
    out = torch.empty((rows, 128), dtype=tdt[do], device="cuda")
    lout = torch.empty(rows, dtype=torch.float32, device="cuda")
    mla.mla_merge_states_n(to, di, tl, pieces, rows, out, do, lout)
    to2 = to.clone(); tl2 = tl.clone()
    mla.mla_merge_states_n(to2, di, tl2, pieces, rows, to2[0], di, tl2[0])
    torch.cuda.synchronize()
    go = f64(to)
    # fold from the merge identity (0, -inf), so that a single empty piece
    # also gives (0, -inf)
    ref_o, ref_l = np.zeros((rows, 128)), np.full(rows, -np.inf)
    for p in range(pieces):
        ref_o, ref_l = orc.merge_states(ref_o, ref_l, go[p], lse[p].astype(np.float64))
    tol = 1e-5 if do == 2 else 2 ** -8
    got = f64(out)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref_o) / np.maximum(np.abs(ref_o), 1.0)) <= tol
    check_lse(f64(lout), ref_l, tol=1e-5)
    assert np.all(got[:5] == 0.0)
    if di == do:
        assert torch.equal(to2[0], out) and torch.equal(tl2[0], lout)


@pytest.mark.parametrize("di", [0, 2])
def test_merge_states_sets(di):
    """mla_merge_states_sets: four merges in one launch (64, 3, 36 and 9
    pieces; 1031, 70, 513 and 0 rows) give each set exactly what
    mla_merge_states_n gives it alone (a set with fewer pieces than the
    launch's wavefronts folds its pieces in the same order), and match the
    oracle's pairwise merge folded over the pieces."""
    require_gpu()
    rng = np.random.default_rng(46 + di)
    tdt = {0: torch.bfloat16, 2: torch.float32}
    sets, alone = [], []
    for pieces, rows in [(64, 1031), (3, 70), (36, 513), (9, 0)]:
        o = rng.standard_normal((pieces, max(rows, 1), 128)).astype(np.float32)
        lse = (rng.standard_normal((pieces, max(rows, 1))) * 3 + 8).astype(np.float32)
        lse[:, :2] = -np.inf                          # every piece empty
        lse[0, 2:9] = -np.inf                         # some pieces empty
        to = torch.tensor(o).to(tdt[di]).cuda()
        tl = torch.tensor(lse).cuda()
        out = torch.full((max(rows, 1), 128), 7.0, dtype=torch.bfloat16, device="cuda")
        lout = torch.full((max(rows, 1),), 7.0, dtype=torch.float32, device="cuda")
        ref = torch.empty_like(out); refl = torch.empty_like(lout)
        mla.mla_merge_states_n(to, di, tl, pieces, rows, ref, 0, refl)
        sets.append((to, tl, pieces, rows, out, lout))
        alone.append((ref, refl, o, lse))
    mla.mla_merge_states_sets(sets, di, 0)
    torch.cuda.synchronize()
    for (to, tl, pieces, rows, out, lout), (ref, refl, o, lse) in zip(sets, alone):
        if rows == 0:
            assert bool((out == 7.0).all()) and bool((lout == 7.0).all())
            continue
        assert torch.equal(out, ref) and torch.equal(lout, refl), f"{pieces} pieces"
        go = f64(to)
        ref_o, ref_l = np.zeros((rows, 128)), np.full(rows, -np.inf)
        for p in range(pieces):
            ref_o, ref_l = orc.merge_states(ref_o, ref_l, go[p], lse[p].astype(np.float64))
        got = f64(out)
        assert np.max(np.abs(got - ref_o) / np.maximum(np.abs(ref_o), 1.0)) <= 2 ** -8
        check_lse(f64(lout), ref_l, tol=1e-5)


# ---------------------------------------------------------------- rope relocation

@pytest.mark.parametrize("delta", [0, 1, 4096, 2 ** 18])
@pytest.mark.parametrize("pairing", [0, 1])
def test_rope_relocate(delta, pairing):
    require_gpu()
    rng = np.random.default_rng(44)
    T, H = 37, 5
    q = mi.f32_to_bf16_bits(rng.standard_normal((T, H, 192)).astype(np.float32))
    tq = bf16_dev(q)
    tout = torch.empty_like(tq)
    mla.mla_rope_relocate_q(tq, tout, H * 192, T, H, delta, 10000.0, pairing)
    tin = tq.clone()
    mla.mla_rope_relocate_q(tin, tin, H * 192, T, H, delta, 10000.0, pairing)
    torch.cuda.synchronize()
    ref = orc.relocate_q(orc.bf16_to_f64(q[..., 128:]), delta, pairing="interleaved" if pairing == 0 else "half")
    got = f64(tout)
    assert np.array_equal(bits(tout)[..., :128], q[..., :128])       # nope part copied
    err = np.abs(got[..., 128:] - ref)
    assert np.all(err <= 2 ** -8 * np.maximum(np.abs(ref), 2 ** -6) + 1e-6)
    assert torch.equal(tin, tout)                                     # in place == out of place
    assert np.array_equal(bits(tq), q)                                # input untouched


# ---------------------------------------------------------------- decompression

# The last two cases give every workgroup of the persistent grid several
# tiles (363 and 528 tiles of 256 x 256), the first of them with an odd head
# count, so one tile straddles the W_UK / W_UV boundary.
@pytest.mark.parametrize("H,h0,h1,n", [(8, 0, 8, 300), (4, 1, 3, 129), (2, 0, 2, 1),
                                       (16, 3, 14, 8300), (16, 0, 16, 8250)])
def test_decompress(H, h0, h1, n):
    require_gpu()
    say(f"decompress H={H} heads [{h0},{h1}) n={n}")
    rng = np.random.default_rng(45)
    lat = mi.f32_to_bf16_bits(rng.standard_normal((n, 576)).astype(np.float32))
    W = mi.f32_to_bf16_bits((rng.standard_normal((512, H * 256)) / math.sqrt(512)).astype(np.float32))
    w_t = pf.pack_weight(W, "cuda")
    Hs = h1 - h0
    hst = (n + 3) * 128
    k = torch.zeros((Hs, n + 3, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((Hs, n + 3, 128), dtype=torch.bfloat16, device="cuda")
    mla.mla_decompress(bf16_dev(lat), 576, None, n, w_t, H, h0, h1, k, hst, v, hst)
    torch.cuda.synchronize()
    # packing itself is exact
    assert np.array_equal(bits(w_t), W.T)
    Wf = orc.bf16_to_f64(W)
    C = orc.bf16_to_f64(lat[:, :512])
    for hs, h in enumerate(range(h0, h1)):
        kr, vr = orc.decompress_head(C, Wf, H, h)
        # the bar, and per element: one bf16 rounding of an fp32 sum of 512
        # products, |got - ref| <= U |ref| + 1.01 GAMMA sum_i |c_i w_i|
        ka, va = orc.decompress_head(np.abs(C), np.abs(Wf), H, h)
        for name, got, ref, absum in (("k", k, kr, ka), ("v", v, vr, va)):
            g = f64(got[hs, :n])
            check_out(g, ref, what=f"{name} head {h}")
            bound = U_BF16 * np.abs(ref) + 1.01 * GAMMA_512 * absum
            bad = np.abs(g - ref) > bound
            assert not bad.any(), f"{name} head {h}: {int(bad.sum())} elements beyond the rounding bound"
        assert np.all(f64(k[hs, n:]) == 0) and np.all(f64(v[hs, n:]) == 0)   # no write past n


def _fp8_rows(rng, n, codes_kind):
    """n latent rows of 1152 bytes whose first 512 bytes are E4M3FN codes
    (every finite code, or random finite codes), rope elements 512..575 bf16,
    bytes 512..1023 poisoned (0xFF: NaN codes, never to be read), and fp32
    scales."""
    rows = np.full((n, 1152), 0xFF, dtype=np.uint8)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    if codes_kind == "all":
        codes = np.stack([np.roll(np.resize(finite, 512), 5 * i) for i in range(n)])
    else:
        codes = rng.choice(finite, size=(n, 512))
    rows[:, :512] = codes
    rows[:, 1024:] = np.frombuffer(mi.f32_to_bf16_bits(rng.standard_normal((n, 64)).astype(np.float32)).tobytes(),
                                   dtype=np.uint8).reshape(n, 128)
    scales = (np.exp(rng.uniform(-6, 2, size=n)) / 448).astype(np.float32)
    return rows, codes, scales


@pytest.mark.parametrize("H,h0,h1,n", [(4, 0, 4, 300), (16, 3, 14, 8300)])
def test_decompress_fp8_rows(H, h0, h1, n):
    """mla_decompress with row_scale: the A rows are E4M3FN codes and the
    scale multiplies the fp32 sums. Random weights: the bar and the
    per-element rounding bound against the exact dequantised product."""
    require_gpu()
    say(f"decompress fp8 rows H={H} heads [{h0},{h1}) n={n}")
    rng = np.random.default_rng(46)
    rows, codes, scales = _fp8_rows(rng, n, "random")
    W = mi.f32_to_bf16_bits((rng.standard_normal((512, H * 256)) / math.sqrt(512)).astype(np.float32))
    w_t = pf.pack_weight(W, "cuda")
    Hs = h1 - h0
    hst = (n + 3) * 128
    k = torch.zeros((Hs, n + 3, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((Hs, n + 3, 128), dtype=torch.bfloat16, device="cuda")
    mla.mla_decompress(torch.from_numpy(rows).cuda(), 576, torch.from_numpy(scales).cuda(), n, w_t, H, h0, h1,
                       k, hst, v, hst)
    torch.cuda.synchronize()
    Wf = orc.bf16_to_f64(W)
    C = orc.e4m3fn_to_f64(codes) * scales.astype(np.float64)[:, None]
    for hs, h in enumerate(range(h0, h1)):
        kr, vr = orc.decompress_head(C, Wf, H, h)
        ka, va = orc.decompress_head(np.abs(C), np.abs(Wf), H, h)
        for name, got, ref, absum in (("k", k, kr, ka), ("v", v, vr, va)):
            g = f64(got[hs, :n])
            check_out(g, ref, what=f"{name} head {h}")
            # fp32 sum of the exact products, one fp32 product with the
            # scale, one bf16 rounding
            bound = U_BF16 * np.abs(ref) + 1.01 * (GAMMA_512 + 2.0 ** -24) * absum
            bad = np.abs(g - ref) > bound
            assert not bad.any(), f"{name} head {h}: {int(bad.sum())} elements beyond the rounding bound"
        assert np.all(f64(k[hs, n:]) == 0) and np.all(f64(v[hs, n:]) == 0)


def test_decompress_fp8_rows_exact():
    """Every finite E4M3FN code through a selection kv_b_proj: each output is
    one code times a power of two times the scale, which the GPU rounds to
    fp32 once and to bf16 once; the oracle does the same two roundings."""
    require_gpu()
    rng = np.random.default_rng(47)
    H, n = 4, 200
    rows, codes, scales = _fp8_rows(rng, n, "all")
    W = mi.selection_kv_b_proj(rng, H)
    w_t = pf.pack_weight(W, "cuda")
    k = torch.empty((H, n, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((H, n, 128), dtype=torch.bfloat16, device="cuda")
    mla.mla_decompress(torch.from_numpy(rows).cuda(), 576, torch.from_numpy(scales).cuda(), n, w_t, H, 0, H,
                       k, n * 128, v, n * 128)
    torch.cuda.synchronize()
    Wf = orc.bf16_to_f64(W)
    Cx = orc.e4m3fn_to_f64(codes)                 # code values: the products with W are exact
    for h in range(H):
        kr, vr = orc.decompress_head(Cx, Wf, H, h)
        for name, got, ref in (("k", k, kr), ("v", v, vr)):
            exp = orc.f32_to_bf16_bits_rne(orc.f64_to_f32_rne(ref * scales.astype(np.float64)[:, None]))
            # equal values (a zero's sign depends on the order of the zero terms)
            assert np.array_equal(f64(got[h]), orc.bf16_to_f64(exp)), f"{name} head {h}"


def test_gather_fp8_raw_bit_exact():
    require_gpu()
    prob = mi.make_problem(4, [256, 64 * 7, 0, 128], [1, 1, 1, 1], 128, "fp8", seed=41, extra_blocks=5, poison=True)
    pool = pf.upload_pool(prob, "cuda")
    bt = _i32(prob.block_table)
    starts = np.array([3, 70, 0, 64]); lens = np.array([250, 301, 0, 64])
    cu = np.concatenate([[0], np.cumsum(lens)])
    out = torch.full((int(cu[-1]) + 1, 576), -7.0, dtype=torch.bfloat16, device="cuda")
    sc = torch.full((int(cu[-1]) + 1,), -3.0, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mla.mla_gather_context_fp8_raw(pool, prob.num_blocks, bt, bt.shape[1], _i32(starts), _i32(lens), _i32(cu), 4,
                                   int(lens.max()), out, sc, status)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.uint8).numpy()          # [rows, 1152] bytes
    gs = sc.cpu().numpy()
    for r in range(4):
        codes, rope, scl = orc.gather_fp8_raw(prob.pool, prob.block_table, r, int(starts[r]), int(lens[r]))
        rows = slice(cu[r], cu[r + 1])
        assert np.array_equal(got[rows, :512], codes), f"request {r} codes"
        assert np.array_equal(got[rows, 1024:].view(np.uint16), rope), f"request {r} rope"
        assert np.array_equal(gs[rows].view(np.uint32), scl.view(np.uint32)), f"request {r} scales"
        # bytes 512..1023 are not written
        assert np.all(got[rows, 512:1024].view(np.uint16) == bits(torch.tensor([-7.0], dtype=torch.bfloat16))[0])
    assert np.all(f64(out[-1]) == -7.0) and gs[-1] == -3.0
    assert int(status.item()) == 0


# ---------------------------------------------------------------- attention

def _attn_case(seed, H, h0, h1, nq, nk, causal, out_dtype, row_ids=False):
    rng = np.random.default_rng(seed)
    B = len(nq)
    Hs = h1 - h0
    cu_q = np.concatenate([[0], np.cumsum(nq)]); cu_k = np.concatenate([[0], np.cumsum(nk)])
    NK = int(cu_k[-1])
    Tphys = int(cu_q[-1]) + 9
    q = mi.f32_to_bf16_bits(rng.standard_normal((Tphys, H, 192)).astype(np.float32))
    kn = mi.f32_to_bf16_bits(rng.standard_normal((Hs, max(NK, 1), 128)).astype(np.float32))
    v = mi.f32_to_bf16_bits(rng.standard_normal((Hs, max(NK, 1), 128)).astype(np.float32))
    lat = mi.f32_to_bf16_bits(rng.standard_normal((max(NK, 1), 576)).astype(np.float32))
    rid = rng.permutation(Tphys)[:int(cu_q[-1])].astype(np.int32) if row_ids else None
    T = int(cu_q[-1])
    scale = 1 / math.sqrt(192)
    odt = torch.float32 if out_dtype == mla.DTYPE_FP32 else torch.bfloat16
    out = torch.full((T, Hs, 128), 9.0, dtype=odt, device="cuda")
    lse = torch.full((T, Hs), 9.0, dtype=torch.float32, device="cuda")
    hst = max(NK, 1) * 128
    mla.mla_prefill_attn(bf16_dev(q), H * 192, H, h0, h1, bf16_dev(kn), hst, bf16_dev(v), hst,
                         bf16_dev(lat), 576, _i32(cu_q), _i32(cu_k),
                         None if rid is None else _i32(rid), B, int(max(nq)), scale, int(causal),
                         out, out_dtype, Hs * 128, lse, Hs)
    torch.cuda.synchronize()
    go, gl = f64(out), f64(lse)
    worst = (0.0, 0.0, 0.0)
    for b in range(B):
        rows = np.arange(cu_q[b], cu_q[b + 1])
        prow = rid[rows] if rid is not None else rows
        keys = np.arange(cu_k[b], cu_k[b + 1])
        vis = orc.causal_visible(nq[b], nk[b] - nq[b]) if causal else None
        for hs, h in enumerate(range(h0, h1)):
            ro, rl = orc.attend(orc.bf16_to_f64(q[prow, h]), orc.bf16_to_f64(kn[hs, keys]),
                                orc.bf16_to_f64(lat[keys, 512:]), orc.bf16_to_f64(v[hs, keys]), scale, vis)
            ma, r = check_out(go[rows, hs], ro, what=f"b{b} h{h} out")
            le = check_lse(gl[rows, hs], rl, what=f"b{b} h{h} lse")
            worst = tuple(max(x, y) for x, y in zip(worst, (ma, r, le)))
    say(f"  attn worst max-abs {worst[0]:.2e} rel-L2 {worst[1]:.2e} lse {worst[2]:.2e}")


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("out_dtype", [mla.DTYPE_BF16, mla.DTYPE_FP32])
def test_attention_varlen(causal, out_dtype):
    require_gpu()
    say(f"attn varlen causal={causal} out={out_dtype}")
    # several query tiles (128 rows each), ragged tails, an empty request
    nq = [300, 1, 0, 77]
    nk = [300 + 130, 1, 5, 77] if causal else [700, 64, 5, 0]
    _attn_case(50 + causal, 3, 0, 3, nq, nk, causal, out_dtype)


@pytest.mark.parametrize("nq", [[64], [100], [40, 64], [300, 77]])
def test_attention_row_ids_and_head_range(nq):
    require_gpu()
    say(f"attn row ids nq={nq}")
    _attn_case(60, 6, 2, 5, nq, [513] * len(nq), 0, mla.DTYPE_FP32, row_ids=True)


def test_attention_empty_keys_give_zero_and_neg_inf():
    require_gpu()
    _attn_case(61, 2, 0, 2, [33, 5], [0, 0], 0, mla.DTYPE_BF16)


# ---------------------------------------------------------------- attention merged into a state

@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("in_place", [True, False])
def test_attention_merge_into_previous_state(causal, in_place):
    """Keys of every request split into a first segment (attended alone, fp32
    state) and a second one attended with mla_prefill_attn_merge against that
    state; the result must be the attention over all keys. With causal = 1 the
    second segment is the request's own new tokens (bottom-right causal), as
    in the chunk loop. Empty segments on either side exercise the -inf rules."""
    require_gpu()
    say(f"attn merge causal={causal} in_place={in_place}")
    rng = np.random.default_rng(70 + causal)
    H, h0, h1 = 3, 0, 3
    Hs = h1 - h0
    nq = [300, 5, 0, 77, 40]
    if causal:
        nA = [300, 0, 5, 130, 0]            # context keys
        nB = list(nq)                       # the new tokens themselves
    else:
        nA = [0, 64, 3, 100, 0]
        nB = [700, 0, 2, 0, 0]
    B = len(nq)
    cu_q = np.concatenate([[0], np.cumsum(nq)])
    T = int(cu_q[-1])
    q = mi.f32_to_bf16_bits(rng.standard_normal((T, H, 192)).astype(np.float32))
    scale = 1 / math.sqrt(192)

    def segment(n):
        cu = np.concatenate([[0], np.cumsum(n)]); NK = max(int(cu[-1]), 1)
        kn = mi.f32_to_bf16_bits(rng.standard_normal((Hs, NK, 128)).astype(np.float32))
        v = mi.f32_to_bf16_bits(rng.standard_normal((Hs, NK, 128)).astype(np.float32))
        lat = mi.f32_to_bf16_bits(rng.standard_normal((NK, 576)).astype(np.float32))
        return cu, NK, kn, v, lat

    cuA, NKA, knA, vA, latA = segment(nA)
    cuB, NKB, knB, vB, latB = segment(nB)
    acc = torch.full((T, Hs, 128), float("nan"), dtype=torch.float32, device="cuda")
    accl = torch.full((T, Hs), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_prefill_attn(bf16_dev(q), H * 192, H, h0, h1, bf16_dev(knA), NKA * 128, bf16_dev(vA), NKA * 128,
                         bf16_dev(latA), 576, _i32(cu_q), _i32(cuA), None, B, max(nq), scale, 0,
                         acc, mla.DTYPE_FP32, Hs * 128, accl, Hs)
    if in_place:
        out, odt, lse = acc, mla.DTYPE_FP32, accl
    else:
        out = torch.full((T, Hs, 128), 9.0, dtype=torch.bfloat16, device="cuda")
        odt = mla.DTYPE_BF16
        lse = torch.full((T, Hs), 9.0, dtype=torch.float32, device="cuda")
    mla.mla_prefill_attn_merge(bf16_dev(q), H * 192, H, h0, h1, bf16_dev(knB), NKB * 128, bf16_dev(vB),
                               NKB * 128, bf16_dev(latB), 576, _i32(cu_q), _i32(cuB), None, B, max(nq),
                               scale, causal, acc, Hs * 128, accl, Hs, out, odt, Hs * 128, lse, Hs)
    torch.cuda.synchronize()
    go, gl = f64(out), f64(lse)
    for b in range(B):
        rows = np.arange(cu_q[b], cu_q[b + 1])
        ka = np.arange(cuA[b], cuA[b + 1]); kb = np.arange(cuB[b], cuB[b + 1])
        vis = orc.causal_visible(nq[b], nA[b]) if causal else None
        for hs in range(Hs):
            kn = np.concatenate([knA[hs, ka], knB[hs, kb]]); vv = np.concatenate([vA[hs, ka], vB[hs, kb]])
            kr = np.concatenate([latA[ka, 512:], latB[kb, 512:]])
            ro, rl = orc.attend(orc.bf16_to_f64(q[rows, h0 + hs]), orc.bf16_to_f64(kn), orc.bf16_to_f64(kr),
                                orc.bf16_to_f64(vv), scale, vis)
            check_out(go[rows, hs], ro, what=f"b{b} h{hs} out")
            # k_nope and v are given to kernel and oracle alike: the bar holds
            # for every row, however few keys it sees
            check_lse(gl[rows, hs], rl, tol=LSE_ABS, what=f"b{b} h{hs} lse")


# ---------------------------------------------------------------- two key segments in one pass

# (seed, nq, nA, nB, merge): nA plain keys (the last context chunk), nB causal
# keys (the request's new tokens: row i sees key j <= i + nB - nq), merged
# into a previous state from nC further plain keys when `merge`. max_q above
# 64 gives 128-row tiles (4 wavefronts) with ragged last tiles, max_q <= 64
# gives 64-row tiles; empty segments on either side; one request with
# nB != nq.
TWO_SEG_CASES = [
    (80, [300, 5, 0, 77, 40, 260], [700, 0, 5, 130, 0, 64], [300, 5, 0, 77, 43, 260], True),
    (81, [300, 5, 0, 77, 40, 260], [700, 0, 5, 130, 0, 64], [300, 5, 0, 77, 43, 260], False),
    (82, [100, 64, 7], [256, 0, 65], [100, 64, 7], True),
    (83, [33, 64, 1], [0, 129, 3], [33, 64, 1], True),
]


@pytest.mark.parametrize("case", TWO_SEG_CASES, ids=[f"seed{c[0]}" for c in TWO_SEG_CASES])
def test_attention_two_segments(case):
    """mla_prefill_attn_2seg: the last chunk's keys and the new tokens' keys
    (causal) in one pass, merged into a state holding further keys; the
    result must be the plain softmax over all three key sets."""
    require_gpu()
    seed, nq, nA, nB, merge = case
    say(f"attn two segments seed={seed} nq={nq} merge={merge}")
    rng = np.random.default_rng(seed)
    H, h0, h1 = 3, 0, 3
    Hs = h1 - h0
    nC = [int(x) for x in rng.integers(0, 200, len(nq))] if merge else [0] * len(nq)
    B = len(nq)
    cu_q = np.concatenate([[0], np.cumsum(nq)])
    T = int(cu_q[-1])
    q = mi.f32_to_bf16_bits(rng.standard_normal((T, H, 192)).astype(np.float32))
    scale = 1 / math.sqrt(192)

    def segment(n):
        cu = np.concatenate([[0], np.cumsum(n)]); NK = max(int(cu[-1]), 1)
        kn = mi.f32_to_bf16_bits(rng.standard_normal((Hs, NK, 128)).astype(np.float32))
        v = mi.f32_to_bf16_bits(rng.standard_normal((Hs, NK, 128)).astype(np.float32))
        lat = mi.f32_to_bf16_bits(rng.standard_normal((NK, 576)).astype(np.float32))
        return cu, NK, kn, v, lat

    cuA, NKA, knA, vA, latA = segment(nA)
    cuB, NKB, knB, vB, latB = segment(nB)
    cuC, NKC, knC, vC, latC = segment(nC)
    acc = accl = None
    if merge:
        acc = torch.full((T, Hs, 128), float("nan"), dtype=torch.float32, device="cuda")
        accl = torch.full((T, Hs), float("nan"), dtype=torch.float32, device="cuda")
        mla.mla_prefill_attn(bf16_dev(q), H * 192, H, h0, h1, bf16_dev(knC), NKC * 128, bf16_dev(vC),
                             NKC * 128, bf16_dev(latC), 576, _i32(cu_q), _i32(cuC), None, B, max(nq), scale, 0,
                             acc, mla.DTYPE_FP32, Hs * 128, accl, Hs)
    out = torch.full((T, Hs, 128), 9.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, Hs), 9.0, dtype=torch.float32, device="cuda")
    mla.mla_prefill_attn_2seg(bf16_dev(q), H * 192, H, h0, h1, bf16_dev(knA), NKA * 128, bf16_dev(vA),
                              NKA * 128, bf16_dev(latA), 576, _i32(cuA), bf16_dev(knB), NKB * 128,
                              bf16_dev(vB), NKB * 128, bf16_dev(latB), 576, _i32(cuB), _i32(cu_q), B,
                              max(nq), scale, acc, Hs * 128, accl, Hs, out, mla.DTYPE_BF16, Hs * 128, lse, Hs)
    torch.cuda.synchronize()
    go, gl = f64(out), f64(lse)
    for b in range(B):
        rows = np.arange(cu_q[b], cu_q[b + 1])
        kc = np.arange(cuC[b], cuC[b + 1]); ka = np.arange(cuA[b], cuA[b + 1]); kb = np.arange(cuB[b], cuB[b + 1])
        # keys C and A all visible; key j of B visible to row i iff j <= i + nB - nq
        i = np.arange(nq[b])[:, None]
        vis = np.concatenate([np.ones((nq[b], len(kc) + len(ka)), dtype=bool),
                              np.arange(nB[b])[None, :] <= i + nB[b] - nq[b]], axis=1)
        for hs in range(Hs):
            kn = np.concatenate([knC[hs, kc], knA[hs, ka], knB[hs, kb]])
            vv = np.concatenate([vC[hs, kc], vA[hs, ka], vB[hs, kb]])
            kr = np.concatenate([latC[kc, 512:], latA[ka, 512:], latB[kb, 512:]])
            ro, rl = orc.attend(orc.bf16_to_f64(q[rows, h0 + hs]), orc.bf16_to_f64(kn), orc.bf16_to_f64(kr),
                                orc.bf16_to_f64(vv), scale, vis)
            check_out(go[rows, hs], ro, what=f"b{b} h{hs} out")
            check_lse(gl[rows, hs], rl, tol=LSE_ABS, what=f"b{b} h{hs} lse")


# ---------------------------------------------------------------- one chunk pass with per-request last flags

# (seed, nq, nA, nB, last, merge): nA plain keys (this chunk), nB causal keys
# (the new tokens, taken only where last[b]), a previous state from nC
# further keys when `merge`. Requests with last[b] == 0 and no key in this
# chunk: in a merging pass their state is left as it was; in a first pass
# they get the empty state (0, -inf).
CHUNK_PASS_CASES = [
    (90, [300, 5, 0, 77, 40, 260], [700, 0, 5, 130, 0, 64], [300, 5, 0, 77, 43, 260], [1, 0, 1, 0, 0, 1], True),
    (91, [300, 5, 0, 77, 40, 260], [700, 3, 5, 130, 9, 64], [300, 5, 0, 77, 43, 260], [0, 1, 1, 0, 1, 1], False),
    (92, [100, 64, 7], [256, 0, 65], [100, 64, 7], [0, 1, 1], True),
    (93, [33, 64, 1], [0, 129, 3], [33, 64, 1], [0, 0, 1], False),
]


@pytest.mark.parametrize("case", CHUNK_PASS_CASES, ids=[f"seed{c[0]}" for c in CHUNK_PASS_CASES])
def test_attention_chunk_pass(case):
    """mla_prefill_attn_chunk: requests whose last chunk this is take the new
    tokens' keys (causal) too and get their final bf16 result (lse into the
    state's lse); the others' running fp32 state is written or merged into.
    Each row is checked against the plain softmax over its key sets, and
    whatever a row must not write is checked unchanged, bit for bit."""
    require_gpu()
    seed, nq, nA, nB, last, merge = case
    say(f"attn chunk pass seed={seed} nq={nq} last={last} merge={merge}")
    # odd seeds take a head range that starts past head 0 (q holds 4 heads)
    H, h0, h1 = (3, 0, 3) if seed % 2 == 0 else (4, 1, 4)
    check_chunk_pass(seed, nq, nA, nB, last, merge, H, h0, h1)


def check_chunk_pass(seed, nq, nA, nB, last, merge, H, h0, h1):
    """mla_prefill_attn_chunk on seeded inputs against the oracle, and the
    rows each route must leave alone unchanged (see test_attention_chunk_pass)."""
    rng = np.random.default_rng(seed)
    Hs = h1 - h0
    nC = [int(x) for x in rng.integers(1, 200, len(nq))] if merge else [0] * len(nq)
    B = len(nq)
    cu_q = np.concatenate([[0], np.cumsum(nq)])
    T = int(cu_q[-1])
    q = mi.f32_to_bf16_bits(rng.standard_normal((T, H, 192)).astype(np.float32))
    scale = 1 / math.sqrt(192)

    def segment(n):
        cu = np.concatenate([[0], np.cumsum(n)]); NK = max(int(cu[-1]), 1)
        kn = mi.f32_to_bf16_bits(rng.standard_normal((Hs, NK, 128)).astype(np.float32))
        v = mi.f32_to_bf16_bits(rng.standard_normal((Hs, NK, 128)).astype(np.float32))
        lat = mi.f32_to_bf16_bits(rng.standard_normal((NK, 576)).astype(np.float32))
        return cu, NK, kn, v, lat

    cuA, NKA, knA, vA, latA = segment(nA)
    cuB, NKB, knB, vB, latB = segment(nB)
    cuC, NKC, knC, vC, latC = segment(nC)
    acc = torch.full((T, Hs, 128), float("nan"), dtype=torch.float32, device="cuda")
    accl = torch.full((T, Hs), float("nan"), dtype=torch.float32, device="cuda")
    if merge:
        mla.mla_prefill_attn(bf16_dev(q), H * 192, H, h0, h1, bf16_dev(knC), NKC * 128, bf16_dev(vC),
                             NKC * 128, bf16_dev(latC), 576, _i32(cu_q), _i32(cuC), None, B, max(nq), scale, 0,
                             acc, mla.DTYPE_FP32, Hs * 128, accl, Hs)
    torch.cuda.synchronize()
    acc0, accl0 = acc.clone(), accl.clone()
    out = torch.full((T, Hs, 128), 9.0, dtype=torch.bfloat16, device="cuda")
    mla.mla_prefill_attn_chunk(bf16_dev(q), H * 192, H, h0, h1, bf16_dev(knA), NKA * 128, bf16_dev(vA),
                               NKA * 128, bf16_dev(latA), 576, _i32(cuA), bf16_dev(knB), NKB * 128,
                               bf16_dev(vB), NKB * 128, bf16_dev(latB), 576, _i32(cuB), _i32(last),
                               _i32(cu_q), B, max(nq), scale, merge, acc, Hs * 128, accl, Hs, out, Hs * 128)
    torch.cuda.synchronize()

    def same_bits(a, b):
        return torch.equal(a.view(torch.int32), b.view(torch.int32))

    go, ga, gl = f64(out), f64(acc), f64(accl)
    for b in range(B):
        rows = np.arange(cu_q[b], cu_q[b + 1])
        r = slice(int(cu_q[b]), int(cu_q[b + 1]))
        kc = np.arange(cuC[b], cuC[b + 1]); ka = np.arange(cuA[b], cuA[b + 1])
        kb = np.arange(cuB[b], cuB[b + 1]) if last[b] else np.arange(0)
        if not last[b] and merge and nA[b] == 0:
            assert same_bits(acc[r], acc0[r]) and same_bits(accl[r], accl0[r]), f"b{b}: state changed"
            assert bool((out[r] == 9.0).all()), f"b{b}: out written"
            continue
        i = np.arange(nq[b])[:, None]
        vis = np.concatenate([np.ones((nq[b], len(kc) + len(ka)), dtype=bool),
                              np.arange(len(kb))[None, :] <= i + len(kb) - nq[b]], axis=1)
        for hs in range(Hs):
            kn = np.concatenate([knC[hs, kc], knA[hs, ka], knB[hs, kb]])
            vv = np.concatenate([vC[hs, kc], vA[hs, ka], vB[hs, kb]])
            kr = np.concatenate([latC[kc, 512:], latA[ka, 512:], latB[kb, 512:]])
            ro, rl = orc.attend(orc.bf16_to_f64(q[rows, h0 + hs]), orc.bf16_to_f64(kn), orc.bf16_to_f64(kr),
                                orc.bf16_to_f64(vv), scale, vis)
            res = go if last[b] else ga
            check_out(res[rows, hs], ro, what=f"b{b} h{hs} {'out' if last[b] else 'state'}")
            check_lse(gl[rows, hs], rl, tol=LSE_ABS, what=f"b{b} h{hs} lse")
        if last[b]:
            # the final rows leave the fp32 state as it was
            assert same_bits(acc[r], acc0[r]), f"b{b}: state written"
        else:
            assert bool((out[r] == 9.0).all()), f"b{b}: out written"


# ---------------------------------------------------------------- absorbed-form attention

@pytest.mark.parametrize("n_rows,pieces", [(37, [0, 300, 364, 1000, 1000]), (64, [0, 2048]), (130, [0, 31, 97]),
                                           (70, [0, 100, 100, 250, 400, 401, 700, 900, 1100, 1300])])
def test_absorbed_path(n_rows, pieces):
    """mla_absorb_q -> mla_absorbed_attn over key pieces (ragged, a 64-key
    piece, an empty one, a one-key one) -> the pieces merged with
    mla_merge_states as four 128-wide states per row -> mla_absorb_out,
    against the oracle's absorbed definition per head over all keys; each
    piece's (o_lat, lse) is also checked against the plain softmax over that
    piece. The last case has 9 pieces of 3 row tiles: 27 work items in
    per-XCD ranges of 4, so ranges cut pieces at several places."""
    require_gpu()
    say(f"absorbed path rows={n_rows} pieces={pieces}")
    rng = np.random.default_rng(75 + n_rows)
    H, h0, h1, Tphys = 8, 2, 7, max(200, n_rows + 10)
    Hs = h1 - h0
    NK = pieces[-1]
    q = mi.f32_to_bf16_bits(rng.standard_normal((Tphys, H, 192)).astype(np.float32))
    lat = mi.f32_to_bf16_bits(rng.standard_normal((max(NK, 1) + 3, 576)).astype(np.float32))
    # With few keys the final lse is compared over a handful of scores, so a
    # selection kv_b_proj keeps the absorbed query exact in bf16 (a rounded
    # q_abs would move those scores by up to ~5e-2); with more keys a random one
    few = NK < 256
    W = (mi.selection_kv_b_proj(rng, H) if few else
         mi.f32_to_bf16_bits((rng.standard_normal((512, H * 256)) / math.sqrt(512)).astype(np.float32)))
    rid = np.sort(rng.choice(Tphys, n_rows, replace=False)).astype(np.int32)
    scale = 1 / math.sqrt(192)
    R = Hs * n_rows
    qa = torch.empty((R, 576), dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q(bf16_dev(q), H * 192, H, h0, h1, _i32(rid), n_rows, bf16_dev(W), H, qa)
    P = len(pieces) - 1
    o_lat = torch.full((P * R, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse4 = torch.full((P * R, 4), float("nan"), dtype=torch.float32, device="cuda")
    dlat = bf16_dev(lat)
    mla.mla_absorbed_attn(qa, R, dlat, 576, _i32(pieces), P, scale, o_lat, mla.DTYPE_FP32, lse4)
    torch.cuda.synchronize()
    qa_h = bits(qa)
    Wf = orc.bf16_to_f64(W)
    # q_abs against the definition
    for hs, h in enumerate(range(h0, h1)):
        ref = orc.bf16_to_f64(q[rid, h, :128]) @ Wf[:, h * 128:(h + 1) * 128].T
        check_out(orc.bf16_to_f64(qa_h[hs * n_rows:(hs + 1) * n_rows, :512]), ref, what=f"q_abs head {h}")
        assert np.array_equal(qa_h[hs * n_rows:(hs + 1) * n_rows, 512:], q[rid, h, 128:])
    # every piece is a plain softmax over its keys, with the kernel's own q_abs
    L = orc.bf16_to_f64(lat)
    QA = orc.bf16_to_f64(qa_h)
    go, gl = f64(o_lat), f64(lse4)
    for b in range(P):
        keys = np.arange(pieces[b], pieces[b + 1])
        if len(keys):
            sc = scale * (QA @ L[keys].T)
            m = sc.max(axis=1)
            e = np.exp(sc - m[:, None])
            ro, rl = (e @ L[keys, :512]) / e.sum(axis=1)[:, None], m + np.log(e.sum(axis=1))
        else:
            ro, rl = np.zeros((R, 512)), np.full(R, -np.inf)
        check_out(go[b * R:(b + 1) * R], ro, what=f"piece {b} o_lat")
        for k4 in range(4):
            check_lse(gl[b * R:(b + 1) * R, k4], rl, tol=LSE_ABS, what=f"piece {b} lse[{k4}]")
    # merge the pieces (first half with last half, in place; the last level to bf16)
    n = P
    fin = torch.empty((R, 512), dtype=torch.bfloat16, device="cuda")
    finl = torch.empty((R, 4), dtype=torch.float32, device="cuda")
    if n == 1:   # a single piece: the attention writes the bf16 state itself
        mla.mla_absorbed_attn(qa, R, dlat, 576, _i32(pieces), 1, scale, fin, mla.DTYPE_BF16, finl)
    while n > 1:
        hh = n // 2; m0 = n - hh
        a, al = o_lat[:hh * R], lse4[:hh * R]
        bb, bl = o_lat[m0 * R:], lse4[m0 * R:]
        if n == 2:
            mla.mla_merge_states(a, mla.DTYPE_FP32, al, bb, mla.DTYPE_FP32, bl, hh * R * 4, fin, mla.DTYPE_BF16, finl)
        else:
            mla.mla_merge_states(a, mla.DTYPE_FP32, al, bb, mla.DTYPE_FP32, bl, hh * R * 4, a, mla.DTYPE_FP32, al)
        n = m0
    wt = pf.pack_weight(W, "cuda")
    out = torch.full((n_rows, Hs * 128), 7.0, dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_out(fin, n_rows, wt, H, h0, h1, out, Hs * 128)
    torch.cuda.synchronize()
    got = f64(out)
    for hs, h in enumerate(range(h0, h1)):
        ro, rl = orc.attend_absorbed(orc.bf16_to_f64(q[rid, h]), L[:NK], Wf, H, h, scale)
        check_out(got[:, hs * 128:(hs + 1) * 128], ro, what=f"out head {h}")
        if few:
            # the exact absorbed query: the kernel's q_abs equals the definition
            ref_qa = orc.bf16_to_f64(q[rid, h, :128]) @ Wf[:, h * 128:(h + 1) * 128].T
            assert np.array_equal(orc.bf16_to_f64(qa_h[hs * n_rows:(hs + 1) * n_rows, :512]), ref_qa)
        check_lse(f64(finl)[hs * n_rows:(hs + 1) * n_rows, 0], rl, tol=LSE_ABS, what=f"lse head {h}")


# ---------------------------------------------------------------- head partition merge

# (T, HL, HG, P, d_mid, d_model): the first gives few 128-wide tiles, so the
# launcher takes 64-wide ones; the second gives 17 x 16 = 272 128-wide tiles,
# at least one per compute unit, so it takes those (ragged last row tile)
@pytest.mark.parametrize("shape", [(300, 7, 1, 13, 256, 384), (2100, 7, 1, 40, 2048, 2048)])
def test_head_partition_merge(shape):
    require_gpu()
    say(f"head partition merge {shape}")
    rng = np.random.default_rng(62)
    T, HL, HG, P, d_mid, d_model = shape
    art = mi.f32_to_bf16_bits(rng.standard_normal((T, HL, 128)).astype(np.float32) * 0.05)
    rec = mi.f32_to_bf16_bits(rng.standard_normal((P, HL, 128)).astype(np.float32) * 0.05)
    glob = mi.f32_to_bf16_bits(rng.standard_normal((T, HG, 128)).astype(np.float32) * 0.05)
    prot = np.sort(rng.choice(T, P, replace=False)).astype(np.int32)
    prot[0] = 0; prot[-1] = T - 1
    prot = np.unique(prot)
    P = len(prot); rec = rec[:P]
    WaL = mi.f32_to_bf16_bits((rng.standard_normal((HL * 128, d_mid)) / math.sqrt(HL * 128)).astype(np.float32))
    WaG = mi.f32_to_bf16_bits((rng.standard_normal((HG * 128, d_mid)) / math.sqrt(HG * 128)).astype(np.float32))
    Wb = mi.f32_to_bf16_bits((rng.standard_normal((d_mid, d_model)) / math.sqrt(d_mid)).astype(np.float32))
    wa_t = pf.pack_weight(np.concatenate([WaL, WaG], 0), "cuda")
    wb_t = pf.pack_weight(Wb, "cuda")
    z = torch.empty((T, d_mid), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, d_model), dtype=torch.bfloat16, device="cuda")
    mla.mla_head_partition_merge(bf16_dev(art), bf16_dev(rec), _i32(prot), P, bf16_dev(glob), wa_t, wb_t,
                                 T, HL, HG, d_mid, d_model, z, y)
    torch.cuda.synchronize()
    O_L = orc.replace_protected(orc.bf16_to_f64(art), orc.bf16_to_f64(rec), prot)
    ref = orc.head_partition_merge(O_L, orc.bf16_to_f64(glob), orc.bf16_to_f64(WaL),
                                   orc.bf16_to_f64(WaG), orc.bf16_to_f64(Wb))
    ma, r = check_out(f64(y), ref, what="y")
    say(f"  y max-abs {ma:.2e} rel-L2 {r:.2e}")
    # a missed replacement would show: rows use rec, not art
    wrong = orc.head_partition_merge(orc.bf16_to_f64(art), orc.bf16_to_f64(glob), orc.bf16_to_f64(WaL),
                                     orc.bf16_to_f64(WaG), orc.bf16_to_f64(Wb))
    assert rel_l2(f64(y)[prot], wrong[prot]) > 0.1
