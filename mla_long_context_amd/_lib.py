"""ctypes binding of libmla.so: argument marshalling only.

Every function takes device pointers (ints) or torch tensors (their
data_ptr() is passed) and a stream handle; it raises MlaError when the
library returns a non-zero status. No computation happens here.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_LAUNCH = -3
MLA_ERR_OUT_OF_RANGE = -4

DTYPE_BF16 = 0
DTYPE_FP8_E4M3 = 1
DTYPE_FP32 = 2

ROPE_INTERLEAVED = 0
ROPE_HALF = 1

EXPORTS = (
    "mla_last_error", "mla_abi_version", "mla_gather_context", "mla_gather_context_fp8_raw", "mla_cache_append",
    "mla_pack_weight_t",
    "mla_decompress", "mla_prefill_attn", "mla_prefill_attn_merge", "mla_prefill_attn_2seg", "mla_prefill_attn_chunk",
    "mla_absorb_q",
    "mla_absorbed_attn", "mla_absorb_out", "mla_merge_states", "mla_merge_states_n",
    "mla_merge_states_sets",
    "mla_rope_relocate_q",
    "mla_head_partition_merge", "mla_head_partition_merge_noalloc", "mla_token_hash", "mla_artifact_check",
)

# reasons written by mla_artifact_check
ARTIFACT_VALID = 0
ARTIFACT_MISSING_LAYER = 1
ARTIFACT_TOKEN_MISMATCH = 2
ARTIFACT_PROFILE_MISMATCH = 3
ARTIFACT_STALE = 4
ARTIFACT_REASONS = {0: "valid", 1: "missing layer", 2: "token mismatch", 3: "profile mismatch",
                    4: "stale generation"}


class ArtifactMeta(ctypes.Structure):
    """mla_artifact_meta: description of an offline Local-head artifact, or
    of what a request needs from one (field meanings as in mla.h)."""
    _fields_ = [("generation", ctypes.c_uint64), ("token_hash", ctypes.c_uint64),
                ("n_tokens", ctypes.c_int64), ("n_heads", ctypes.c_int32), ("n_local", ctypes.c_int32),
                ("d_c", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("rope_base", ctypes.c_double), ("n_layers", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("layer_mask", ctypes.c_uint64)]


class MlaMergeSet(ctypes.Structure):
    """One merge of mla_merge_states_sets (field meanings as in mla.h)."""
    _fields_ = [("outs", ctypes.c_void_p), ("lses", ctypes.c_void_p), ("pieces", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("out", ctypes.c_void_p), ("lse_out", ctypes.c_void_p)]


MERGE_MAX_SETS = 4


class MlaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} -> {code}: {msg}")
        self.code = code


DEVICE_STATUS_TEXT = {
    MLA_ERR_OUT_OF_RANGE: "a block id outside the pool (or a position outside the block table) reached "
                          "the device; the records it named were not read (zeros were written in their place)",
}


def raise_on_device_status(code: int, what: str) -> None:
    """Raise MlaError for a device status word read back after a step
    (MLA_OK = 0 passes)."""
    code = int(code)
    if code != MLA_OK:
        raise MlaError(what, code, DEVICE_STATUS_TEXT.get(code, "device-side error"))


_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int
I64 = ctypes.c_int64
F32 = ctypes.c_float
F64 = ctypes.c_double

_SIGS = {
    "mla_gather_context": [P, I32, I32, P, I64, P, P, P, I32, I32, P, P, P],
    "mla_cache_append": [P, I32, I32, P, I64, P, P, I32, I32, P, I64, P, P],
    "mla_pack_weight_t": [P, I32, I32, P, P],
    "mla_gather_context_fp8_raw": [P, I32, P, I64, P, P, P, I32, I32, P, P, P, P],
    "mla_decompress": [P, I64, P, I32, P, I32, I32, I32, P, I64, P, I64, P],
    "mla_prefill_attn": [P, I64, I32, I32, I32, P, I64, P, I64, P, I64, P, P, P,
                         I32, I32, F32, I32, P, I32, I64, P, I64, P],
    "mla_prefill_attn_merge": [P, I64, I32, I32, I32, P, I64, P, I64, P, I64, P, P, P,
                               I32, I32, F32, I32, P, I64, P, I64, P, I32, I64, P, I64, P],
    "mla_prefill_attn_2seg": [P, I64, I32, I32, I32, P, I64, P, I64, P, I64, P,
                              P, I64, P, I64, P, I64, P, P, I32, I32, F32,
                              P, I64, P, I64, P, I32, I64, P, I64, P],
    "mla_prefill_attn_chunk": [P, I64, I32, I32, I32, P, I64, P, I64, P, I64, P,
                               P, I64, P, I64, P, I64, P, P, P, I32, I32, F32,
                               I32, P, I64, P, I64, P, I64, P],
    "mla_absorb_q": [P, I64, I32, I32, I32, P, I32, P, I32, P, P],
    "mla_absorbed_attn": [P, I32, P, I64, P, I32, F32, P, I32, P, P],
    "mla_absorb_out": [P, I32, P, I32, I32, I32, P, I64, P],
    "mla_merge_states": [P, I32, P, P, I32, P, I64, P, I32, P, P],
    "mla_merge_states_n": [P, I32, P, I32, I64, P, I32, P, P],
    "mla_merge_states_sets": [P, I32, I32, I32, P],
    "mla_rope_relocate_q": [P, P, I64, I32, I32, I64, F64, I32, P],
    "mla_head_partition_merge": [P, P, P, I32, P, P, P, I32, I32, I32, I32, I32, P, P, P],
    "mla_head_partition_merge_noalloc": [P, P, P, I32, P, P, P, I32, I32, I32, I32, I32, P, P],
    "mla_artifact_check": [ctypes.POINTER(ArtifactMeta), ctypes.POINTER(ArtifactMeta), ctypes.POINTER(I32)],
}


def load(path: str = LIB_PATH):
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m mla_long_context_amd.build`")
    lib = ctypes.CDLL(path)
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_abi_version.restype = I32
    lib.mla_abi_version.argtypes = []
    lib.mla_token_hash.restype = ctypes.c_uint64
    lib.mla_token_hash.argtypes = [P, I64]
    for name, args in _SIGS.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = I32
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _call(name, *args):
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != MLA_OK:
        raise MlaError(name, rc, lib.mla_last_error().decode())
    return rc


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def mla_gather_context(pool, cache_dtype, num_blocks, block_table, bt_stride, chunk_start,
                       chunk_len, cu_out, batch, max_len, out_latent, dev_status=None, stream=None):
    return _call("mla_gather_context", _ptr(pool), cache_dtype, num_blocks, _ptr(block_table),
                 bt_stride, _ptr(chunk_start), _ptr(chunk_len), _ptr(cu_out), batch, max_len,
                 _ptr(out_latent), _ptr(dev_status), _stream(stream))


def mla_cache_append(pool, cache_dtype, num_blocks, block_table, bt_stride, pos0, cu_new, batch,
                     max_new, latent_new, ld_latent, dev_status=None, stream=None):
    return _call("mla_cache_append", _ptr(pool), cache_dtype, num_blocks, _ptr(block_table),
                 bt_stride, _ptr(pos0), _ptr(cu_new), batch, max_new, _ptr(latent_new), ld_latent,
                 _ptr(dev_status), _stream(stream))


def mla_pack_weight_t(w, K, N, out, stream=None):
    return _call("mla_pack_weight_t", _ptr(w), K, N, _ptr(out), _stream(stream))


def mla_decompress(latent, ld_latent, row_scale, n_tokens, w_t, H_total, h_begin, h_end, k_nope,
                   k_head_stride, v, v_head_stride, stream=None):
    return _call("mla_decompress", _ptr(latent), ld_latent, _ptr(row_scale), n_tokens, _ptr(w_t), H_total,
                 h_begin, h_end, _ptr(k_nope), k_head_stride, _ptr(v), v_head_stride, _stream(stream))


def mla_gather_context_fp8_raw(pool, num_blocks, block_table, bt_stride, chunk_start, chunk_len, cu_out, batch,
                               max_len, out_latent, out_scale, dev_status=None, stream=None):
    return _call("mla_gather_context_fp8_raw", _ptr(pool), num_blocks, _ptr(block_table), bt_stride,
                 _ptr(chunk_start), _ptr(chunk_len), _ptr(cu_out), batch, max_len, _ptr(out_latent),
                 _ptr(out_scale), _ptr(dev_status), _stream(stream))


def mla_prefill_attn(q, q_row_stride, H_q, h_begin, h_end, k_nope, k_head_stride, v,
                     v_head_stride, latent, ld_latent, cu_q, cu_k, q_row_ids, batch, max_q,
                     scale, causal, out, out_dtype, out_row_stride, lse, lse_row_stride,
                     stream=None):
    return _call("mla_prefill_attn", _ptr(q), q_row_stride, H_q, h_begin, h_end, _ptr(k_nope),
                 k_head_stride, _ptr(v), v_head_stride, _ptr(latent), ld_latent, _ptr(cu_q),
                 _ptr(cu_k), _ptr(q_row_ids), batch, max_q, float(scale), int(causal), _ptr(out),
                 out_dtype, out_row_stride, _ptr(lse), lse_row_stride, _stream(stream))


def mla_prefill_attn_merge(q, q_row_stride, H_q, h_begin, h_end, k_nope, k_head_stride, v,
                           v_head_stride, latent, ld_latent, cu_q, cu_k, q_row_ids, batch, max_q,
                           scale, causal, prev_out, prev_row_stride, prev_lse, prev_lse_row_stride,
                           out, out_dtype, out_row_stride, lse, lse_row_stride, stream=None):
    return _call("mla_prefill_attn_merge", _ptr(q), q_row_stride, H_q, h_begin, h_end, _ptr(k_nope),
                 k_head_stride, _ptr(v), v_head_stride, _ptr(latent), ld_latent, _ptr(cu_q),
                 _ptr(cu_k), _ptr(q_row_ids), batch, max_q, float(scale), int(causal), _ptr(prev_out),
                 prev_row_stride, _ptr(prev_lse), prev_lse_row_stride, _ptr(out), out_dtype,
                 out_row_stride, _ptr(lse), lse_row_stride, _stream(stream))


def mla_prefill_attn_2seg(q, q_row_stride, H_q, h_begin, h_end, k_nope, k_head_stride, v,
                          v_head_stride, latent, ld_latent, cu_k, k_nope2, k_head_stride2, v2,
                          v_head_stride2, latent2, ld_latent2, cu_k2, cu_q, batch, max_q, scale,
                          prev_out, prev_row_stride, prev_lse, prev_lse_row_stride, out, out_dtype,
                          out_row_stride, lse, lse_row_stride, stream=None):
    return _call("mla_prefill_attn_2seg", _ptr(q), q_row_stride, H_q, h_begin, h_end, _ptr(k_nope),
                 k_head_stride, _ptr(v), v_head_stride, _ptr(latent), ld_latent, _ptr(cu_k),
                 _ptr(k_nope2), k_head_stride2, _ptr(v2), v_head_stride2, _ptr(latent2), ld_latent2,
                 _ptr(cu_k2), _ptr(cu_q), batch, max_q, float(scale), _ptr(prev_out), prev_row_stride,
                 _ptr(prev_lse), prev_lse_row_stride, _ptr(out), out_dtype, out_row_stride, _ptr(lse),
                 lse_row_stride, _stream(stream))


def mla_prefill_attn_chunk(q, q_row_stride, H_q, h_begin, h_end, k_nope, k_head_stride, v,
                           v_head_stride, latent, ld_latent, cu_k, k_nope2, k_head_stride2, v2,
                           v_head_stride2, latent2, ld_latent2, cu_k2, last, cu_q, batch, max_q, scale,
                           merge, state, state_row_stride, state_lse, state_lse_row_stride, out,
                           out_row_stride, stream=None):
    return _call("mla_prefill_attn_chunk", _ptr(q), q_row_stride, H_q, h_begin, h_end, _ptr(k_nope),
                 k_head_stride, _ptr(v), v_head_stride, _ptr(latent), ld_latent, _ptr(cu_k),
                 _ptr(k_nope2), k_head_stride2, _ptr(v2), v_head_stride2, _ptr(latent2), ld_latent2,
                 _ptr(cu_k2), _ptr(last), _ptr(cu_q), batch, max_q, float(scale), int(merge),
                 _ptr(state), state_row_stride, _ptr(state_lse), state_lse_row_stride, _ptr(out),
                 out_row_stride, _stream(stream))


def mla_absorb_q(q, q_row_stride, H_q, h_begin, h_end, row_ids, n_rows, kv_b_proj, H_total, q_abs,
                 stream=None):
    return _call("mla_absorb_q", _ptr(q), q_row_stride, H_q, h_begin, h_end, _ptr(row_ids), n_rows,
                 _ptr(kv_b_proj), H_total, _ptr(q_abs), _stream(stream))


def mla_absorbed_attn(q_abs, R, latent, ld_latent, cu_k, pieces, scale, out_lat, out_dtype, lse4,
                      stream=None):
    return _call("mla_absorbed_attn", _ptr(q_abs), R, _ptr(latent), ld_latent, _ptr(cu_k), pieces,
                 float(scale), _ptr(out_lat), out_dtype, _ptr(lse4), _stream(stream))


def mla_absorb_out(o_lat, n_rows, w_t, H_total, h_begin, h_end, out, out_row_stride, stream=None):
    return _call("mla_absorb_out", _ptr(o_lat), n_rows, _ptr(w_t), H_total, h_begin, h_end, _ptr(out),
                 out_row_stride, _stream(stream))


def mla_merge_states(out_a, dtype_a, lse_a, out_b, dtype_b, lse_b, rows, out, dtype_out, lse_out,
                     stream=None):
    return _call("mla_merge_states", _ptr(out_a), dtype_a, _ptr(lse_a), _ptr(out_b), dtype_b,
                 _ptr(lse_b), rows, _ptr(out), dtype_out, _ptr(lse_out), _stream(stream))


def mla_merge_states_n(outs, dtype_in, lses, pieces, rows, out, dtype_out, lse_out, stream=None):
    return _call("mla_merge_states_n", _ptr(outs), dtype_in, _ptr(lses), pieces, rows, _ptr(out), dtype_out,
                 _ptr(lse_out), _stream(stream))


def mla_merge_states_sets(sets, dtype_in, dtype_out, stream=None):
    """sets: (outs, lses, pieces, rows, out, lse_out) per merge, at most
    MERGE_MAX_SETS of them."""
    arr = (MlaMergeSet * max(len(sets), 1))()
    for i, (outs, lses, pieces, rows, out, lse_out) in enumerate(sets):
        arr[i] = MlaMergeSet(_ptr(outs), _ptr(lses), pieces, rows, _ptr(out), _ptr(lse_out))
    return _call("mla_merge_states_sets", ctypes.cast(arr, ctypes.c_void_p), len(sets), dtype_in, dtype_out,
                 _stream(stream))


def mla_rope_relocate_q(q_in, q_out, q_row_stride, T, H, delta, rope_base=10000.0,
                        pairing=ROPE_INTERLEAVED, stream=None):
    return _call("mla_rope_relocate_q", _ptr(q_in), _ptr(q_out), q_row_stride, T, H, int(delta),
                 float(rope_base), pairing, _stream(stream))


def mla_head_partition_merge(art_out, rec_out, prot_rows, P, glob_out, wa_t, wb_t, T, HL, HG,
                             d_mid, d_model, z, y, stream=None):
    return _call("mla_head_partition_merge", _ptr(art_out), _ptr(rec_out), _ptr(prot_rows), P,
                 _ptr(glob_out), _ptr(wa_t), _ptr(wb_t), T, HL, HG, d_mid, d_model, _ptr(z),
                 _ptr(y), _stream(stream))


def mla_head_partition_merge_noalloc(art_out, rec_out, prot_rows, P, glob_out, wa_t, wb_t, T, HL, HG,
                                     d_mid, d_model, y, stream=None):
    return _call("mla_head_partition_merge_noalloc", _ptr(art_out), _ptr(rec_out), _ptr(prot_rows), P,
                 _ptr(glob_out), _ptr(wa_t), _ptr(wb_t), T, HL, HG, d_mid, d_model, _ptr(y), _stream(stream))


def mla_token_hash(tokens) -> int:
    """64-bit FNV-1a of int32 token ids (a host array-like)."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    return int(load().mla_token_hash(a.ctypes.data if a.size else None, a.size))


def mla_artifact_check(artifact: ArtifactMeta, request: ArtifactMeta) -> int:
    """First failing validation check (ARTIFACT_* reason), host only."""
    reason = I32(-1)
    _call("mla_artifact_check", ctypes.byref(artifact), ctypes.byref(request), ctypes.byref(reason))
    return reason.value
