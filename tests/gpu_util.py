"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import os
import sys

import numpy as np
import pytest
import torch

# tolerances for floating-point outputs against the fp64 oracle
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
LSE_ABS = 1e-3
FP8_REL_L2 = 2e-2
# Edge-case problems (not the standard workloads): rows that see fewer than
# FEW_KEYS keys have an lse dominated by a handful of scores. A score's error
# from rounding a decompressed key to bf16 (unit roundoff 2^-8) is up to
# scale * 2^-8 * sum_d |q_d k_d|, about 2.3e-2 for N(0,1) data at d = 128 (an
# fp8 cache adds the same again from rounding the dequantised latent), and
# with few keys it is not averaged away. Such rows are held to LSE_FEW_KEYS;
# every row of the standard workloads sees >= 257 keys and is held to LSE_ABS.
FEW_KEYS = 256
LSE_FEW_KEYS = 3e-2


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
