"""The C-ABI library loads without a GPU, exports every entry point the header
declares, and rejects bad arguments on the host before anything is enqueued
(these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

import mla_long_context_amd as mla
from mla_long_context_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "mla.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmla.so is not built (python -m mla_long_context_amd.build)")
    return mla.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert len(declared) >= 9
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)
    assert lib.mla_abi_version() == 2


def _err(fn, *args):
    with pytest.raises(mla.MlaError) as ei:
        fn(*args, stream=0)
    return ei.value.code, str(ei.value)


FAKE = 1 << 20      # a 16-byte aligned non-null "device pointer" never dereferenced


def test_gather_validation(lib):
    code, msg = _err(mla.mla_gather_context, None, 0, 4, FAKE, 4, FAKE, FAKE, FAKE, 1, 64, FAKE, None)
    assert code == _lib.MLA_ERR_INVALID_ARG and "null" in msg
    code, _ = _err(mla.mla_gather_context, FAKE, 7, 4, FAKE, 4, FAKE, FAKE, FAKE, 1, 64, FAKE, None)
    assert code == _lib.MLA_ERR_UNSUPPORTED
    code, _ = _err(mla.mla_gather_context, FAKE + 2, 0, 4, FAKE, 4, FAKE, FAKE, FAKE, 1, 64, FAKE, None)
    assert code == _lib.MLA_ERR_INVALID_ARG
    code, _ = _err(mla.mla_gather_context, FAKE, 0, 0, FAKE, 4, FAKE, FAKE, FAKE, 1, 64, FAKE, None)
    assert code == _lib.MLA_ERR_INVALID_ARG
    # empty work is a no-op, even with null pointers
    assert mla.mla_gather_context(None, 0, 0, None, 0, None, None, None, 0, 0, None, None, stream=0) == 0


def test_decompress_validation(lib):
    code, _ = _err(mla.mla_decompress, FAKE, 576, None, 10, FAKE, 8, 3, 3, FAKE, 1280, FAKE, 1280)
    assert code == _lib.MLA_ERR_INVALID_ARG                      # empty head range
    code, _ = _err(mla.mla_decompress, FAKE, 576, None, 10, FAKE, 8, 0, 9, FAKE, 1280, FAKE, 1280)
    assert code == _lib.MLA_ERR_INVALID_ARG                      # h_end > H
    code, _ = _err(mla.mla_decompress, FAKE, 500, None, 10, FAKE, 8, 0, 8, FAKE, 1280, FAKE, 1280)
    assert code == _lib.MLA_ERR_INVALID_ARG                      # ld < 512
    code, _ = _err(mla.mla_decompress, FAKE, 576, None, 10, FAKE, 8, 0, 8, FAKE, 1000, FAKE, 1280)
    assert code == _lib.MLA_ERR_INVALID_ARG                      # head stride too small
    code, _ = _err(mla.mla_decompress, FAKE, 576, FAKE + 2, 10, FAKE, 8, 0, 8, FAKE, 1280, FAKE, 1280)
    assert code == _lib.MLA_ERR_INVALID_ARG                      # misaligned row_scale
    assert mla.mla_decompress(None, 576, None, 0, None, 8, 0, 8, None, 0, None, 0, stream=0) == 0
    code, msg = _err(mla.mla_gather_context_fp8_raw, FAKE, 4, FAKE, 4, FAKE, FAKE, FAKE, 1, 64, FAKE, None, None)
    assert code == _lib.MLA_ERR_INVALID_ARG and "null" in msg    # no scale output
    assert mla.mla_gather_context_fp8_raw(None, 0, None, 0, None, None, None, 0, 0, None, None, stream=0) == 0


def test_attn_validation(lib):
    base = [FAKE, 8 * 192, 8, 0, 8, FAKE, 1280, FAKE, 1280, FAKE, 576, FAKE, FAKE, None, 1, 10,
            0.07, 0, FAKE, 0, 8 * 128, FAKE, 8]
    args = list(base); args[19] = 5
    assert _err(mla.mla_prefill_attn, *args)[0] == _lib.MLA_ERR_UNSUPPORTED
    args = list(base); args[1] = 8 * 192 - 8
    assert _err(mla.mla_prefill_attn, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    args = list(base); args[16] = -1.0
    assert _err(mla.mla_prefill_attn, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    args = list(base); args[0] = None
    assert _err(mla.mla_prefill_attn, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    args = list(base); args[10] = 512
    assert _err(mla.mla_prefill_attn, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    args = list(base); args[20] = 100
    assert _err(mla.mla_prefill_attn, *args)[0] == _lib.MLA_ERR_INVALID_ARG


def test_two_segment_attn_validation(lib):
    # q, q_rs, H_q, h0, h1, k, khs, v, vhs, lat, ld, cu_k, k2, khs2, v2, vhs2, lat2, ld2, cu_k2, cu_q,
    # batch, max_q, scale, prev_out, prev_rs, prev_lse, prev_lse_rs, out, out_dt, out_rs, lse, lse_rs
    base = [FAKE, 8 * 192, 8, 0, 8, FAKE, 1280, FAKE, 1280, FAKE, 576, FAKE,
            FAKE, 1280, FAKE, 1280, FAKE, 576, FAKE, FAKE, 1, 10, 0.07,
            None, 0, None, 0, FAKE, 0, 8 * 128, FAKE, 8]
    args = list(base); args[17] = 584                     # latents with different row strides
    assert _err(mla.mla_prefill_attn_2seg, *args)[0] == _lib.MLA_ERR_UNSUPPORTED
    args = list(base); args[12] = None                    # no second-segment keys
    code, msg = _err(mla.mla_prefill_attn_2seg, *args)
    assert code == _lib.MLA_ERR_INVALID_ARG and "second-segment" in msg
    args = list(base); args[16] = FAKE + 4                # misaligned second latent
    assert _err(mla.mla_prefill_attn_2seg, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    args = list(base); args[13] = 1284                    # head stride not a multiple of 8
    assert _err(mla.mla_prefill_attn_2seg, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    args = list(base); args[23] = FAKE                    # previous out without its lse
    code, msg = _err(mla.mla_prefill_attn_2seg, *args)
    assert code == _lib.MLA_ERR_INVALID_ARG and "previous state" in msg
    args = list(base); args[20] = 0                       # nothing to do
    assert mla.mla_prefill_attn_2seg(*args, stream=0) == 0


def test_chunk_pass_attn_validation(lib):
    # q, q_rs, H_q, h0, h1, k, khs, v, vhs, lat, ld, cu_k, k2, khs2, v2, vhs2, lat2, ld2, cu_k2, last, cu_q,
    # batch, max_q, scale, merge, state, state_rs, state_lse, state_lse_rs, out, out_rs
    base = [FAKE, 8 * 192, 8, 0, 8, FAKE, 1280, FAKE, 1280, FAKE, 576, FAKE,
            FAKE, 1280, FAKE, 1280, FAKE, 576, FAKE, FAKE, FAKE, 1, 10, 0.07,
            1, FAKE, 8 * 128, FAKE, 8, FAKE, 8 * 128]
    for i, what in [(19, "last"), (25, "state"), (27, "state_lse")]:
        args = list(base); args[i] = None
        code, msg = _err(mla.mla_prefill_attn_chunk, *args)
        assert code == _lib.MLA_ERR_INVALID_ARG and "null" in msg, (what, msg)
    args = list(base); args[26] = 8 * 128 - 4             # state rows narrower than the heads
    code, msg = _err(mla.mla_prefill_attn_chunk, *args)
    assert code == _lib.MLA_ERR_INVALID_ARG and "state" in msg
    args = list(base); args[25] = FAKE + 4                # misaligned state
    assert _err(mla.mla_prefill_attn_chunk, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    args = list(base); args[17] = 584                     # latents with different row strides
    assert _err(mla.mla_prefill_attn_chunk, *args)[0] == _lib.MLA_ERR_UNSUPPORTED
    args = list(base); args[21] = 0                       # nothing to do
    assert mla.mla_prefill_attn_chunk(*args, stream=0) == 0


def test_merge_rope_partition_pack_validation(lib):
    assert _err(mla.mla_merge_states, FAKE, 9, FAKE, FAKE, 0, FAKE, 4, FAKE, 0, FAKE)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert _err(mla.mla_merge_states, FAKE, 0, FAKE, FAKE + 4, 0, FAKE, 4, FAKE, 0, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG
    assert mla.mla_merge_states(None, 0, None, None, 0, None, 0, None, 0, None, stream=0) == 0
    assert _err(mla.mla_merge_states_n, FAKE, 0, FAKE, 0, 4, FAKE, 0, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG  # no piece
    assert _err(mla.mla_merge_states_n, FAKE, 7, FAKE, 3, 4, FAKE, 0, FAKE)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert _err(mla.mla_merge_states_n, FAKE + 8, 0, FAKE, 3, 4, FAKE, 0, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG
    assert mla.mla_merge_states_n(None, 0, None, 3, 0, None, 0, None, stream=0) == 0
    assert _err(mla.mla_rope_relocate_q, FAKE, FAKE, 8 * 192, 4, 8, 4096, 10000.0, 3)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert _err(mla.mla_rope_relocate_q, FAKE, FAKE, 100, 4, 8, 4096, 10000.0, 0)[0] == _lib.MLA_ERR_INVALID_ARG
    assert _err(mla.mla_rope_relocate_q, FAKE, FAKE, 8 * 192, 4, 8, 4096, 0.5, 0)[0] == _lib.MLA_ERR_INVALID_ARG
    assert _err(mla.mla_head_partition_merge, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 16, 7, 1, 2000,
                4096, FAKE, FAKE)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert _err(mla.mla_head_partition_merge, FAKE, FAKE, FAKE, 20, FAKE, FAKE, FAKE, 16, 7, 1, 2048,
                4096, FAKE, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG          # P > T
    assert _err(mla.mla_pack_weight_t, FAKE, 10, 16, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG
    assert _err(mla.mla_pack_weight_t, FAKE, 16, 16, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG   # in place
    # several merges in one launch: at most four sets, each checked as alone
    S = (FAKE, FAKE, 3, 4, FAKE, FAKE)
    assert mla.mla_merge_states_sets([], 0, 0, stream=0) == 0
    assert _err(mla.mla_merge_states_sets, [S] * 5, 0, 0)[0] == _lib.MLA_ERR_INVALID_ARG
    assert _err(mla.mla_merge_states_sets, [S, S], 7, 0)[0] == _lib.MLA_ERR_UNSUPPORTED
    code, msg = _err(mla.mla_merge_states_sets, [S, (FAKE, FAKE, 0, 4, FAKE, FAKE)], 0, 0)
    assert code == _lib.MLA_ERR_INVALID_ARG and "set 1" in msg
    code, msg = _err(mla.mla_merge_states_sets, [S, (FAKE + 8, FAKE, 3, 4, FAKE, FAKE)], 0, 0)
    assert code == _lib.MLA_ERR_INVALID_ARG and "aligned" in msg
    assert mla.mla_merge_states_sets([(None, None, 3, 0, None, None)], 0, 0, stream=0) == 0   # no rows
    # sizes whose grids would not fit the launch limits are refused, not truncated
    for fn, args in [(mla.mla_merge_states, (FAKE, 0, FAKE, FAKE, 0, FAKE, (1 << 34) + 1, FAKE, 0, FAKE)),
                     (mla.mla_rope_relocate_q, (FAKE, FAKE, 1024 * 192, 1 << 25, 1024, 4096, 10000.0, 0))]:
        code, msg = _err(fn, *args)
        assert code == _lib.MLA_ERR_INVALID_ARG and "too large" in msg, msg


def test_last_error_is_thread_local_and_cleared(lib):
    _err(mla.mla_pack_weight_t, FAKE, 10, 16, FAKE)
    assert b"multiples of 8" in lib.mla_last_error()
    assert mla.mla_merge_states(None, 0, None, None, 0, None, 0, None, 0, None, stream=0) == 0
    assert _err(mla.mla_merge_states_n, FAKE, 0, FAKE, 0, 4, FAKE, 0, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG  # no piece
    assert _err(mla.mla_merge_states_n, FAKE, 7, FAKE, 3, 4, FAKE, 0, FAKE)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert _err(mla.mla_merge_states_n, FAKE + 8, 0, FAKE, 3, 4, FAKE, 0, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG
    assert mla.mla_merge_states_n(None, 0, None, 3, 0, None, 0, None, stream=0) == 0
    assert lib.mla_last_error() == b""


# ---------------------------------------------------------------- artifact validation (host only)

def test_token_hash_matches_the_oracle(lib):
    import numpy as np
    from oracle import mla_oracle as orc
    rng = np.random.default_rng(11)
    assert mla.mla_token_hash([]) == orc.artifact_token_hash([]) == 0xcbf29ce484222325
    for n in (1, 2, 7, 1000):
        t = rng.integers(-(1 << 31), 1 << 31, size=n).astype(np.int32)
        assert mla.mla_token_hash(t) == orc.artifact_token_hash(t)


def _meta_pair(rng):
    keys = ("generation", "token_hash", "n_tokens", "n_heads", "n_local", "d_c", "d_rope", "d_nope", "d_v",
            "rope_base", "n_layers", "layer_mask")
    a = dict(generation=int(rng.integers(1, 9)), token_hash=int(rng.integers(0, 1 << 63)),
             n_tokens=int(rng.integers(1, 1 << 20)), n_heads=64, n_local=56, d_c=512, d_rope=64, d_nope=128,
             d_v=128, rope_base=10000.0, n_layers=37, layer_mask=(1 << 37) - 1)
    r = dict(a)
    # perturb a random subset of fields
    for k in keys:
        if rng.random() < 0.15:
            if k == "rope_base":
                r[k] = 50000.0
            elif k == "layer_mask":
                which = int(rng.integers(0, 64))
                if rng.random() < 0.5:
                    a[k] = a[k] & ~(1 << which)
                else:
                    r[k] = r[k] | (1 << which)
            else:
                r[k] = r[k] + 1
    return a, r


def test_artifact_check_matches_the_oracle(lib):
    import numpy as np
    from oracle import mla_oracle as orc
    rng = np.random.default_rng(12)
    seen = set()
    for _ in range(400):
        a, r = _meta_pair(rng)
        want = orc.artifact_check_reason(a, r)
        got = mla.mla_artifact_check(mla.ArtifactMeta(**a), mla.ArtifactMeta(**r))
        assert got == want, (a, r)
        seen.add(want)
    assert seen == {0, 1, 2, 3, 4}


def test_artifact_check_rejects_bad_arguments(lib):
    m = mla.ArtifactMeta(n_layers=65)
    with pytest.raises(mla.MlaError) as ei:
        mla.mla_artifact_check(m, mla.ArtifactMeta())
    assert ei.value.code == _lib.MLA_ERR_INVALID_ARG
    reason = ctypes.c_int(-7)
    assert lib.mla_artifact_check(None, ctypes.byref(mla.ArtifactMeta()), ctypes.byref(reason)) == \
        _lib.MLA_ERR_INVALID_ARG
    assert reason.value == -7


def test_attn_merge_cache_absorbed_validation(lib):
    base = [FAKE, 8 * 192, 8, 0, 8, FAKE, 1280, FAKE, 1280, FAKE, 576, FAKE, FAKE, None, 1, 10,
            0.07, 0, FAKE, 8 * 128, FAKE, 8, FAKE, 2, 8 * 128, FAKE, 8]
    args = list(base); args[18] = None                            # no previous state
    assert _err(mla.mla_prefill_attn_merge, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    args = list(base); args[18] = FAKE + 4                        # misaligned previous state
    assert _err(mla.mla_prefill_attn_merge, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    args = list(base); args[10] = (1 << 17) + 8                   # latent rows too wide
    assert _err(mla.mla_prefill_attn_merge, *args)[0] == _lib.MLA_ERR_INVALID_ARG
    # cache append: dtype, row stride, batch limit; empty work is a no-op
    assert _err(mla.mla_cache_append, FAKE, 7, 4, FAKE, 4, FAKE, FAKE, 1, 8, FAKE, 576, None)[0] == \
        _lib.MLA_ERR_UNSUPPORTED
    assert _err(mla.mla_cache_append, FAKE, 0, 4, FAKE, 4, FAKE, FAKE, 1, 8, FAKE, 512, None)[0] == \
        _lib.MLA_ERR_INVALID_ARG
    assert _err(mla.mla_cache_append, FAKE, 0, 4, FAKE, 4, FAKE, FAKE, 70000, 8, FAKE, 576, None)[0] == \
        _lib.MLA_ERR_INVALID_ARG
    assert mla.mla_cache_append(None, 0, 0, None, 0, None, None, 0, 0, None, 576, None, stream=0) == 0
    # absorbed form: head ranges, dtypes, strides
    assert _err(mla.mla_absorb_q, FAKE, 8 * 192, 8, 3, 3, FAKE, 4, FAKE, 8, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG
    assert _err(mla.mla_absorb_q, FAKE, 8 * 192, 8, 0, 8, FAKE, 4, FAKE, 4, FAKE)[0] == _lib.MLA_ERR_INVALID_ARG
    assert _err(mla.mla_absorbed_attn, FAKE, 4, FAKE, 576, FAKE, 1, 0.07, FAKE, 9, FAKE)[0] == \
        _lib.MLA_ERR_UNSUPPORTED
    assert _err(mla.mla_absorbed_attn, FAKE, 4, FAKE, 500, FAKE, 1, 0.07, FAKE, 0, FAKE)[0] == \
        _lib.MLA_ERR_INVALID_ARG
    assert _err(mla.mla_absorbed_attn, FAKE, 4, FAKE, 576, FAKE, 1, -1.0, FAKE, 0, FAKE)[0] == \
        _lib.MLA_ERR_INVALID_ARG
    assert mla.mla_absorbed_attn(None, 0, None, 576, None, 0, 0.07, None, 0, None, stream=0) == 0
    assert _err(mla.mla_absorb_out, FAKE, 4, FAKE, 8, 0, 8, FAKE, 100)[0] == _lib.MLA_ERR_INVALID_ARG
    assert _err(mla.mla_absorb_out, FAKE, 4, FAKE, 8, 2, 9, FAKE, 1024)[0] == _lib.MLA_ERR_INVALID_ARG


def test_device_status_raises_only_on_error():
    """The drivers' check() turns a non-zero device status word into MlaError
    (the decision is host logic; a GPU test drives it with a bad block id)."""
    _lib.raise_on_device_status(0, "step")
    with pytest.raises(mla.MlaError) as ei:
        _lib.raise_on_device_status(_lib.MLA_ERR_OUT_OF_RANGE, "ChunkedPrefill")
    assert ei.value.code == _lib.MLA_ERR_OUT_OF_RANGE and "outside the pool" in str(ei.value)


def _absorbed_dma_keys(n_k, tile=32, stages=4, rows=32):
    """Host model of the keys the absorbed-attention kernel's DMA reads for a
    piece of n_k keys: the prologue fills stages-1 stages and every step one
    more, each with the tile index clamped to the last tile and every key
    clamped to the last key; an empty piece issues none."""
    ntiles = (n_k + tile - 1) // tile
    keys = set()
    if ntiles > 0:
        for t in list(range(stages - 1)) + [t + stages - 1 for t in range(ntiles)]:
            kt0 = min(t, ntiles - 1) * tile
            keys |= {min(kt0 + r, n_k - 1) for r in range(rows)}
    return keys


@pytest.mark.parametrize("n_k", [0, 1, 31, 32, 33, 100])
def test_absorbed_dma_stays_inside_the_piece(n_k):
    keys = _absorbed_dma_keys(n_k)
    assert all(0 <= k < n_k for k in keys)
    assert keys == set(range(n_k))


def _absorbed_items(pieces, n_rt):
    """Host model of the absorbed-attention launch: the grid is the work
    items (piece, row tile) rounded up to 8 equal per-XCD ranges; workgroup b
    (XCD b % 8, slot b // 8) takes item (b % 8) * per_xcd + b // 8 when that
    is an item."""
    n_items = pieces * n_rt
    per_xcd = (n_items + 7) // 8
    grid = per_xcd * 8
    taken = []
    for b in range(grid):
        slot, item = b >> 3, (b & 7) * per_xcd + (b >> 3)
        if slot < per_xcd and item < n_items:
            taken.append((item // n_rt, item % n_rt, b & 7))
    return taken


@pytest.mark.parametrize("pieces,n_rt", [(1, 1), (1, 28), (8, 28), (9, 28), (36, 28), (3, 5), (17, 1), (2, 129)])
def test_absorbed_work_items_each_once(pieces, n_rt):
    taken = _absorbed_items(pieces, n_rt)
    pairs = [(p, r) for p, r, _ in taken]
    assert sorted(pairs) == [(p, r) for p in range(pieces) for r in range(n_rt)]
    # no XCD gets more than its equal share, and a piece whose row tiles fit
    # in one XCD's range lies on at most two XCDs
    per_xcd = (pieces * n_rt + 7) // 8
    assert max(sum(1 for *_, x in taken if x == k) for k in range(8)) <= per_xcd
    if n_rt <= per_xcd:
        for p in range(pieces):
            assert len({x for q, _, x in taken if q == p}) <= 2


def test_noalloc_merge_rejects_sizes_beyond_its_scratch(lib):
    # T * d_mid above 4194304 bf16 elements is refused before anything else
    code, msg = _err(mla.mla_head_partition_merge_noalloc, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 2049, 7, 1,
                     2048, 128, FAKE)
    assert code == _lib.MLA_ERR_INVALID_ARG and "scratch" in msg
    # an empty call is a no-op
    assert mla.mla_head_partition_merge_noalloc(None, None, None, 0, None, FAKE, FAKE, 0, 7, 1, 2048, 128, FAKE,
                                                stream=0) == 0
