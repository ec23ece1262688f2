"""mla_head_partition_merge_noalloc (z in the library's scratch array, no
allocation) against mla_head_partition_merge with a caller workspace and
against the fp64 oracle: two calls in a row on one device, the first at the
scratch array's full size, the second smaller (the array keeps the first
call's z, which the second must overwrite before reading)."""
import math

import numpy as np
import pytest
import torch

import mla_long_context_amd as mla
from mla_long_context_amd import prefill as pf
from oracle import mla_oracle as orc

from gpu_util import bf16_dev, bits, check_out, f64, require_gpu, say

pytestmark = pytest.mark.gpu


def _case(rng, T, HL, HG, P, d_mid, d_model):
    f = lambda a: orc.bf16_to_f64(a)
    art = _bf16(rng.standard_normal((T, HL, 128)) * 0.05)
    rec = _bf16(rng.standard_normal((P, HL, 128)) * 0.05)
    glob = _bf16(rng.standard_normal((T, HG, 128)) * 0.05)
    prot = np.sort(rng.choice(T, P, replace=False)).astype(np.int32)
    WaL = _bf16(rng.standard_normal((HL * 128, d_mid)) / math.sqrt(HL * 128))
    WaG = _bf16(rng.standard_normal((HG * 128, d_mid)) / math.sqrt(HG * 128))
    Wb = _bf16(rng.standard_normal((d_mid, d_model)) / math.sqrt(d_mid))
    ref = orc.head_partition_merge(orc.replace_protected(f(art), f(rec), prot), f(glob), f(WaL), f(WaG), f(Wb))
    dev = dict(art=bf16_dev(art), rec=bf16_dev(rec), glob=bf16_dev(glob),
               prot=torch.tensor(prot, device="cuda"),
               wa_t=pf.pack_weight(np.concatenate([WaL, WaG], 0), "cuda"), wb_t=pf.pack_weight(Wb, "cuda"))
    return dev, ref


def _bf16(x):
    from mla_inputs import f32_to_bf16_bits
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def test_noalloc_matches_workspace_entry_point_twice():
    require_gpu()
    rng = np.random.default_rng(90)
    # the first call fills the whole scratch array (T * d_mid = 4194304
    # bf16 elements), the second is smaller
    for T, HL, HG, P, d_mid, d_model in [(2048, 7, 1, 40, 2048, 256), (77, 3, 1, 5, 128, 128)]:
        say(f"no-alloc head partition merge T={T} HL={HL} HG={HG} P={P} d_mid={d_mid} d_model={d_model}")
        d, ref = _case(rng, T, HL, HG, P, d_mid, d_model)
        z = torch.empty((T, d_mid), dtype=torch.bfloat16, device="cuda")
        y_ws = torch.full((T, d_model), 7.0, dtype=torch.bfloat16, device="cuda")
        y_na = torch.full((T, d_model), 7.0, dtype=torch.bfloat16, device="cuda")
        mla.mla_head_partition_merge(d["art"], d["rec"], d["prot"], P, d["glob"], d["wa_t"], d["wb_t"], T, HL, HG,
                                     d_mid, d_model, z, y_ws)
        mla.mla_head_partition_merge_noalloc(d["art"], d["rec"], d["prot"], P, d["glob"], d["wa_t"], d["wb_t"], T,
                                             HL, HG, d_mid, d_model, y_na)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: the same bits
        assert np.array_equal(bits(y_na), bits(y_ws))
        ma, r = check_out(f64(y_na), ref, what="y")
        say(f"  y max-abs {ma:.2e} rel-L2 {r:.2e}")


def test_noalloc_rejects_more_than_the_scratch_array():
    require_gpu()
    y = torch.empty((1, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((128, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError) as ei:
        mla.mla_head_partition_merge_noalloc(w, None, None, 0, w, w, w, 2049, 7, 1, 2048, 128, y)
    assert ei.value.code == mla._lib.MLA_ERR_INVALID_ARG and "scratch" in str(ei.value)
