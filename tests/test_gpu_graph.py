"""A step captured into a HIP graph and replayed equals the eager step bit
for bit: every replay, with the program's own eager work and synchronisation
between replays. The kernels are deterministic (no atomics, fixed reduction
orders), so equality is exact."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
from mla_long_context_amd.prefill import ArtifactBuilder, ChunkedPrefill, GraphStep, ReusePrefill

from gpu_util import bits, require_gpu, say

pytestmark = pytest.mark.gpu


def _snap(tensors):
    torch.cuda.synchronize()
    return [bits(t) if t.dtype == torch.bfloat16 else t.detach().cpu().numpy().copy() for t in tensors]


def _same(a, b, what):
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), what


def _check(driver, outputs, what):
    driver.run()
    eager = _snap(outputs(driver))
    g = GraphStep(driver)
    for rep in range(3):
        for t in outputs(driver):
            t.zero_()                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        _same(_snap(outputs(driver)), eager, f"{what}: replay {rep}")
        driver.run()                   # and an eager step
        _same(_snap(outputs(driver)), eager, f"{what}: eager after replay {rep}")


def test_graph_chunked_prefill():
    require_gpu()
    say("graph: chunked prefill (ragged, 3 requests, fp8 and bf16)")
    for dt in ("bf16", "fp8"):
        prob = mi.make_problem(8, [64 * 11, 128, 0], [40, 257, 3], 256, dt, seed=81)
        _check(ChunkedPrefill(prob), lambda d: [d.out, d.lse], f"chunked {dt}")


@pytest.mark.parametrize("local", ["absorbed", "decompressed"])
def test_graph_reuse_prefill(local):
    require_gpu()
    say(f"graph: reuse prefill ({local})")
    prob = mi.make_multidoc_problem(chunk=256)
    _check(ReusePrefill(prob, split=256, split_local=512, local_path=local),
           lambda d: [d.y, d.glob_out, d.lse_G, d.rec_out], f"reuse {local}")


def test_graph_artifact_build():
    require_gpu()
    say("graph: artifact build")
    ap = mi.make_artifact_problem(H=8, n_local=7, L=1088, extra_rows=50, chunk=256, seed=82)
    _check(ArtifactBuilder.from_problem(ap), lambda d: [d.out, d.lse], "artifact")
