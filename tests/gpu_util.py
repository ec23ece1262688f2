"""Helpers shared by the GPU parity tests: comparisons, and tolerance bounds
derived from the oracle's exact values (none of the path's arithmetic)."""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc

# tolerances for floating-point outputs against the fp64 oracle
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
LSE_ABS = 1e-3
FP8_REL_L2 = 2e-2
# Rows of an lse check that see fewer than FEW_KEYS keys with a random
# kv_b_proj take a bound derived from their own data (kv_rounding_lse_bound);
# every other row is held to LSE_ABS. Edge-case problems use a selection
# kv_b_proj (exact decompressed keys) and hold every row to LSE_ABS.
FEW_KEYS = 256
# unit roundoff of bf16 (8 significant bits), and the first-order error
# factor of a 512-term fp32 dot product
U_BF16 = 2.0 ** -8
GAMMA_512 = 512 * 2.0 ** -24
# allowance for the attention kernel's own fp32 arithmetic (scores, exp2,
# sums, log) in a derived lse bound: half the lse bar
ATTN_ALLOW = 5e-4


def kv_rounding_lse_bound(q, c_kv, W, H, h, scale, visible=None, dequant_rounding=False):
    """Bound on |lse_gpu - lse_oracle| per query row of head h when the
    oracle scores the exact decompressed keys k = c_kv W_UK^h and the GPU
    the bf16 ones it stores.

    The GPU key is bf16(fp32 sum): |k~_d - k_d| <= U |k_d| + 1.01 (GAMMA +
    U') sum_i |c_i W_id|, where U' = U when the latent itself was rounded to
    bf16 first (a dequantised fp8 cache) and 0 otherwise. A score moves by at
    most scale * sum_d |q_d| |k~_d - k_d|, and the lse, being 1-Lipschitz in
    the max-norm of the scores, by at most the largest such move over the
    visible keys. q: [R, >=128] fp64 (nope part first), c_kv [N, 512] fp64,
    W [512, H*256] fp64, visible [R, N] bool or None. Returns [R]."""
    q = np.asarray(q, np.float64)
    R = q.shape[0]
    if c_kv.shape[0] == 0:
        return np.full(R, ATTN_ALLOW)
    Wk = W[:, h * 128:(h + 1) * 128]
    k = c_kv @ Wk
    a = np.abs(c_kv) @ np.abs(Wk)
    dk = U_BF16 * np.abs(k) + 1.01 * (GAMMA_512 + (U_BF16 if dequant_rounding else 0.0)) * a
    ds = scale * (np.abs(q[:, :128]) @ dk.T)
    if visible is not None:
        ds = np.where(visible, ds, 0.0)
    return ds.max(axis=1) + ATTN_ALLOW


def relocated_rope_rounding(q_rope, delta, base=10000.0):
    """What the relocation does to a query's rope part, per element, as
    (err, err_max): q_rel - q_rot where the kernel's result is determined
    (err_max 0 there), else 0 and the larger of the two possible |q_rel -
    q_rot|. q_rot is the exact rotation by -delta (interleaved pairs); the
    kernel computes y0 = fma(x0, c, -x1 s), y1 = fma(x0, s, x1 c) in fp32
    with fp32 cos/sin of fp64 angles, within 4 * 2^-24 (|x0| + |x1|) of
    q_rot, and rounds that to bf16 (nearest even). Where the whole interval
    rounds to one bf16 value, that value is q_rel. q_rope: [R, 64] fp64 of
    bf16 values."""
    q = np.asarray(q_rope, np.float64)
    y = orc.relocate_q(q, int(delta), base)
    pair = 4.0 * 2.0 ** -24 * (np.abs(q[:, 0::2]) + np.abs(q[:, 1::2]))
    eps = np.repeat(pair, 2, axis=1)
    from mla_inputs import f32_to_bf16_bits
    lo = orc.bf16_to_f64(f32_to_bf16_bits((y - eps).astype(np.float32)))
    hi = orc.bf16_to_f64(f32_to_bf16_bits((y + eps).astype(np.float32)))
    det = lo == hi
    err = np.where(det, lo - y, 0.0)
    err_max = np.where(det, 0.0, np.maximum(np.abs(lo - y), np.abs(hi - y)))
    return err, err_max


def relocation_lse_bound(prob, q_rows, h):
    """Bound on |lse_gpu - lse_oracle| per query row of head h of a reuse
    problem whose keys are exact (a selection kv_b_proj): the path rotates a
    query's rope part by -delta_d for document d and stores it in bf16, the
    dtype its products take, while the oracle rotates the keys by +delta_d
    exactly. A score against key j of document d then moves by
    scale * (err . k_j) for the determined elements plus at most
    scale * sum err_max |k_j| for the others (relocated_rope_rounding); the
    lse, 1-Lipschitz in the max-norm of the scores, by at most the largest
    such move, plus the attention's own fp32 arithmetic. q_rows: row indices
    into prob.q. Returns [len(q_rows)]."""
    q = orc.bf16_to_f64(prob.q[np.asarray(q_rows), h, 128:])
    bound = np.zeros(len(q))
    for d in prob.documents():
        L = int(d["L"])
        if L == 0:
            continue
        k = orc.bf16_to_f64(orc.gather_bf16_bits(d["pool"], d["block_table"], 0, 0, L))[:, 512:]
        err, err_max = relocated_rope_rounding(q, int(d["delta"]), prob.rope_base)
        ds = prob.scale * (np.abs(err @ k.T) + err_max @ np.abs(k).T)
        bound = np.maximum(bound, ds.max(axis=1) * (1 + 1e-12))
    return bound + ATTN_ALLOW


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a GPU")
    from mla_long_context_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmla.so is not built")
    return "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def bf16_dev(a_bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_bits).view(np.int16)).view(torch.bfloat16).to(device)


def rel_l2(got, ref):
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def check_out(got, ref, max_abs=BF16_MAX_ABS, rl2=BF16_REL_L2, what="out"):
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    ma = float(np.max(np.abs(got - ref))) if got.size else 0.0
    r = rel_l2(got, ref) if got.size else 0.0
    assert ma <= max_abs and r <= rl2, f"{what}: max-abs {ma:.3e} (<= {max_abs}), rel-L2 {r:.3e} (<= {rl2})"
    return ma, r


def check_lse(got, ref, tol=LSE_ABS, what="lse"):
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    ninf_r = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf_r), f"{what}: -inf pattern differs"
    fin = ~ninf_r
    if fin.any():
        tol = np.broadcast_to(np.asarray(tol, np.float64), ref.shape)
        d = np.where(fin, np.abs(np.where(fin, got, 0.0) - np.where(fin, ref, 0.0)), 0.0)
        bad = fin & ~(d <= tol)
        err = float(np.max(d[fin]))
        assert not bad.any(), f"{what}: max-abs {err:.3e} exceeds its tolerance at {np.argwhere(bad)[:4].tolist()}"
        return err
    return 0.0
