"""Plain fp64 CPU oracle for MLA prefill over a paged, packed latent cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
path never routes through it, and it shares no code with the HIP path: it
reads raw input arrays (bf16 bit patterns, E4M3FN codes, fp32) and decodes
them itself.

Every function is the plain definition of what the method computes, written
out in NumPy fp64, with no chunking, paging, blocking or fusion beyond what
that definition states. Pages cited:

* [DSMLA] "DeepSeek MLA -- Prefix Cache and Chunked Prefill" notes:
  section 4.2 (two-stage prefill), 4.3 (merge_attn_states), 4.4
  (_compute_prefill_context chunk loop), 5.2 (packed 576-element buffer),
  section 3 heading (non-absorbed vs absorbed paths).
* [PAGED] "PagedAttention assumed MHA. DeepSeek-V4 says that assumption is
  broken.": sections "What MLA changes about KV cache accounting",
  "Block size is not a tuning knob here", "What DeepSeek-V4 breaks".
* [REDKNOT] "RedKnot-MLA: Multi-Head Offline-Online Reuse for DeepSeek-V4
  Long-Context Serving": Abstract, section 1, section 2 (Equation 4,
  relocation, protected rows), section 3 (runtime consumer).
* Cache write path: [PAGED] "Position independence beats prefix matching"
  (records written into blocks that are sealed when full), [DSMLA] 2.2
  (fp8 storage of the latent; its content is missing from the page, so the
  per-token scale is a reading, R14, stated in quantize_token_e4m3).

Each reading taken where the pages are silent is stated in the docstring of
the function that takes it, under a label R<n>.

Parity unpinned: the synthetic Local-head artifact and the protected-row
choice of the head-partitioned reuse workload are inputs by construction;
no page value checks them. Every function here has a pin in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

D_C = 512
D_ROPE = 64
D_LAT = 576
D_NOPE = 128
D_V = 128
BLOCK = 64
FP8_ROPE_OFF = BLOCK * D_C
FP8_SCALE_OFF = FP8_ROPE_OFF + BLOCK * D_ROPE * 2
NEG_INF = -np.inf


# --------------------------------------------------------------------------
# Number decoding (exact widening to fp64)
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64. bf16 is the top half of an fp32, so the
    widening is a 16-bit shift into fp32 and then an exact fp32->fp64 cast."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes -> fp64, from the bit definition: 1 sign bit, 4
    exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
    (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity (max 448).
    Reading R13: the fp8 cache of the pages uses this OCP variant."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = np.where(e == 0, sub, normal) * sign
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


def f64_to_f32_rne(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 with round to nearest even (NumPy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even on the dropped 16 bits; NaN
    maps to the quiet NaN 0x7FC0."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(x32), np.uint16(0x7FC0), r)


# --------------------------------------------------------------------------
# Paged latent cache: gather by definition
# --------------------------------------------------------------------------

def token_to_slot(block_table: np.ndarray, req: int, t: np.ndarray):
    """Token t of request req lives in physical block block_table[req][t//64]
    at slot t % 64 ([PAGED] "Block size is not a tuning knob here": 64-token
    blocks; [DSMLA] 4.4: the cache is read through a block table; reading
    R11)."""
    t = np.asarray(t, dtype=np.int64)
    return block_table[req, t // BLOCK].astype(np.int64), t % BLOCK


def gather_bf16_bits(pool: np.ndarray, block_table: np.ndarray, req: int,
                     start: int, length: int) -> np.ndarray:
    """Contiguous latent records [length, 576] (bf16 bits) of tokens
    [start, start+length) of a request, from a bf16 pool [NB, 64, 576]
    ([DSMLA] 4.4 step 1; 5.2: each record is c_kv (512) then k_rope (64))."""
    t = np.arange(start, start + length)
    blk, slot = token_to_slot(block_table, req, t)
    return pool[blk, slot, :]


def gather_fp8_f64(pool: np.ndarray, block_table: np.ndarray, req: int,
                   start: int, length: int) -> np.ndarray:
    """Latent records [length, 576] in fp64 from an fp8 pool [NB, 41216]:
    c_kv = decode(code) * scale (exact in fp64: 4 + 24 significant bits),
    k_rope widened from bf16. Layout reading R16: per block, codes [64][512],
    then bf16 rope [64][64], then fp32 scales [64]."""
    t = np.arange(start, start + length)
    blk, slot = token_to_slot(block_table, req, t)
    rows = pool[blk]                                         # [n, 41216]
    codes = rows[np.arange(length)[:, None],
                 slot[:, None] * D_C + np.arange(D_C)[None, :]]
    rope_bytes = rows[:, FP8_ROPE_OFF:FP8_SCALE_OFF].reshape(length, BLOCK, D_ROPE * 2)
    rope_bits = np.ascontiguousarray(rope_bytes[np.arange(length), slot]).view(np.uint16)
    sc_bytes = rows[:, FP8_SCALE_OFF:].reshape(length, BLOCK, 4)
    sc = np.ascontiguousarray(sc_bytes[np.arange(length), slot]).view(np.float32)[:, 0]
    out = np.empty((length, D_LAT), dtype=np.float64)
    out[:, :D_C] = e4m3fn_to_f64(codes) * sc.astype(np.float64)[:, None]
    out[:, D_C:] = bf16_to_f64(rope_bits)
    return out


def gather_fp8_raw(pool: np.ndarray, block_table: np.ndarray, req: int, start: int, length: int):
    """The stored parts of an fp8 cache's records for tokens [start,
    start+length) of a request, as they are in the blocks (layout reading
    R16): codes uint8 [length, 512], k_rope bf16 bits [length, 64], scales
    fp32 [length]. A gather that leaves dequantisation to the decompression
    copies exactly these ([DSMLA] 4.4 step 1 with the fp8 storage of 2.2)."""
    t = np.arange(start, start + length)
    blk, slot = token_to_slot(block_table, req, t)
    rows = pool[blk]
    codes = rows[np.arange(length)[:, None], slot[:, None] * D_C + np.arange(D_C)[None, :]]
    rope = np.ascontiguousarray(rows[:, FP8_ROPE_OFF:FP8_SCALE_OFF].reshape(length, BLOCK, D_ROPE * 2)
                                [np.arange(length), slot]).view(np.uint16)
    sc = np.ascontiguousarray(rows[:, FP8_SCALE_OFF:].reshape(length, BLOCK, 4)[np.arange(length), slot]).view(
        np.float32)[:, 0]
    return codes, rope, sc


def gather_fp8_expected_bits(pool, block_table, req, start, length) -> np.ndarray:
    """The bf16 record a gather that dequantises an fp8 cache must write,
    bit for bit (reading R17): c_kv = bf16_rne(fp32_rne(decode(code) *
    scale)); the fp32 product of two fp32 values is the fp64 exact product
    rounded once to fp32. k_rope bits are copied."""
    x = gather_fp8_f64(pool, block_table, req, start, length)
    bits = np.empty((length, D_LAT), dtype=np.uint16)
    bits[:, :D_C] = f32_to_bf16_bits_rne(f64_to_f32_rne(x[:, :D_C]))
    bits[:, D_C:] = f32_to_bf16_bits_rne(f64_to_f32_rne(x[:, D_C:]))
    return bits


# --------------------------------------------------------------------------
# Cache write path: append new tokens' records into their blocks
# --------------------------------------------------------------------------

def e4m3fn_encode_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 values with |x| <= 448 -> OCP E4M3FN codes, round to nearest even,
    from the bit definition (reading R13): a normal value is (1 + m/8) 2^e
    with e in [-6, 8] and exponent field e + 7; below 2^-6 the code is the
    subnormal m with value m/8 * 2^-6, m = round(|x| * 2^9). A mantissa that
    rounds up to 8 carries into the exponent (for subnormals, m = 8 is the
    smallest normal, code 0x08). The sign bit is the fp32 sign bit, so -0.0
    encodes as 0x80."""
    x = np.asarray(x32, dtype=np.float32)
    assert np.all(np.abs(x) <= 448.0), "encode expects |x| <= 448"
    sign = (x.view(np.uint32) >> np.uint32(31)).astype(np.int64)
    a = np.abs(x).astype(np.float64)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)        # 0..8, exact scaling
    nz = ~sub
    if nz.any():
        e = np.floor(np.log2(a[nz])).astype(np.int64)
        # guard the log2 rounding at exact powers of two
        e = np.where(2.0 ** e > a[nz], e - 1, e)
        e = np.where(2.0 ** (e + 1) <= a[nz], e + 1, e)
        m = np.rint((a[nz] / 2.0 ** e - 1.0) * 8.0).astype(np.int64)  # exact in fp64, then RNE
        carry = m == 8
        e = np.where(carry, e + 1, e)
        m = np.where(carry, 0, m)
        code[nz] = ((e + 7) << 3) | m
    return (code | (sign << 7)).astype(np.uint8)


def quantize_token_e4m3(c_kv_bits: np.ndarray):
    """One fp8 record per token (reading R14): scale = fp32(max|x|) / 448
    rounded once to fp32; code = e4m3_rne(clamp(fp32(x / scale), +-448)).
    Division in fp64 then one rounding to fp32 equals the correctly rounded
    fp32 division (53 >= 2*24 + 2 bits). A row of zeros gets scale 0 and
    +0 codes. Returns (codes uint8 [n, 512], scale fp32 [n])."""
    x = (np.asarray(c_kv_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    amax = np.max(np.abs(x.astype(np.float64)), axis=-1)
    scale = (amax / 448.0).astype(np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    nz = scale > 0
    if nz.any():
        y = (x[nz].astype(np.float64) / scale[nz].astype(np.float64)[:, None]).astype(np.float32)
        codes[nz] = e4m3fn_encode_rne(np.clip(y, np.float32(-448.0), np.float32(448.0)))
    return codes, scale


def cache_append_expected(pool: np.ndarray, block_table: np.ndarray, pos0, lengths,
                          new_bits: np.ndarray, cache_dtype: str) -> np.ndarray:
    """The pool after appending new tokens ([PAGED] "Position independence
    beats prefix matching": records are written into blocks that are sealed
    once full; [DSMLA] 2.2 fp8 storage; reading R16 for the fp8 block
    layout). Token i of request r (rows cu[r] + i of new_bits [n, 576], bf16
    bits) goes to position pos0[r] + i, i.e. block block_table[r][t // 64],
    slot t % 64. bf16 pool [NB, 64, 576]: the record is copied. fp8 pool
    [NB, 41216] bytes: codes and scale from quantize_token_e4m3, rope copied
    as bf16. Nothing else of the pool changes."""
    out = pool.copy()
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    for r in range(len(lengths)):
        n = int(lengths[r])
        if n == 0:
            continue
        t = int(pos0[r]) + np.arange(n)
        blk, slot = token_to_slot(block_table, r, t)
        rec = new_bits[cu[r]:cu[r] + n]
        if cache_dtype == "bf16":
            out[blk, slot, :] = rec
            continue
        codes, scale = quantize_token_e4m3(rec[:, :D_C])
        for j in range(n):
            b, sl = int(blk[j]), int(slot[j])
            out[b, sl * D_C:(sl + 1) * D_C] = codes[j]
            out[b, FP8_ROPE_OFF + sl * D_ROPE * 2:FP8_ROPE_OFF + (sl + 1) * D_ROPE * 2] = \
                np.ascontiguousarray(rec[j, D_C:]).view(np.uint8)
            out[b, FP8_SCALE_OFF + sl * 4:FP8_SCALE_OFF + (sl + 1) * 4] = \
                np.ascontiguousarray(scale[j:j + 1]).view(np.uint8)
    return out


def context_latent_f64(prob, req: int, start: int, length: int) -> np.ndarray:
    """Context latent records of one request in fp64, for either cache dtype."""
    if prob.cache_dtype == "bf16":
        return bf16_to_f64(gather_bf16_bits(prob.pool, prob.block_table, req, start, length))
    return gather_fp8_f64(prob.pool, prob.block_table, req, start, length)


# --------------------------------------------------------------------------
# kv_b_proj decompression ([DSMLA] 4.4 step 2; reading R1)
# --------------------------------------------------------------------------

def decompress_head(c_kv: np.ndarray, W: np.ndarray, H: int, h: int):
    """Per-head keys and values from latents: kv_b_proj W is [512, H*256]
    with all heads' W_UK columns first (head h at h*128) and all heads' W_UV
    columns after (head h at H*128 + h*128). Returns (k_nope [n,128],
    v [n,128]) = (c W_UK^h, c W_UV^h)."""
    Wk = W[:, h * D_NOPE:(h + 1) * D_NOPE]
    Wv = W[:, H * D_NOPE + h * D_V:H * D_NOPE + (h + 1) * D_V]
    return c_kv @ Wk, c_kv @ Wv


# --------------------------------------------------------------------------
# Attention with log-sum-exp ([DSMLA] 4.3, 4.4 steps 3-4)
# --------------------------------------------------------------------------

def attend(q: np.ndarray, k_nope: np.ndarray, k_rope: np.ndarray, v: np.ndarray,
           scale: float, visible: Optional[np.ndarray] = None):
    """Softmax attention of rows q [R,192] (nope 0:128, rope 128:192) for one
    head over keys K = [k_nope | k_rope] ([DSMLA] 4.4 step 3: the rope part
    of the key is shared by every head) and values v.

    s_j = scale * q.K_j over visible j; lse = ln sum_j e^{s_j} (natural log,
    reading R4); out = sum_j softmax(s)_j v_j. A row with no visible key has
    out = 0 and lse = -inf (reading R6)."""
    R = q.shape[0]
    N = k_nope.shape[0]
    if N == 0:
        return np.zeros((R, v.shape[1] if v.ndim == 2 else D_V)), np.full(R, NEG_INF)
    s = scale * (q[:, :D_NOPE] @ k_nope.T + q[:, D_NOPE:] @ k_rope.T)
    if visible is not None:
        s = np.where(visible, s, NEG_INF)
    m = np.max(s, axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    Z = np.sum(e, axis=1)
    Zs = np.where(empty, 1.0, Z)
    out = (e @ v) / Zs[:, None]
    lse = np.where(empty, NEG_INF, m_safe + np.log(Zs))
    out[empty] = 0.0
    return out, lse


def causal_visible(n_rows: int, n_ctx: int) -> np.ndarray:
    """Extend row i (0-based) sees every context key and extend keys j <= i:
    key index k (context first) is visible iff k <= n_ctx + i (reading R7,
    bottom-right alignment)."""
    i = np.arange(n_rows)[:, None]
    k = np.arange(n_ctx + n_rows)[None, :]
    return k <= n_ctx + i


def merge_states(out_a, lse_a, out_b, lse_b):
    """merge_attn_states ([DSMLA] 4.3): m = max(la, lb), w = e^{l-m},
    out = (wa oa + wb ob) / (wa + wb). The merged lse, which the printed
    function omits but the chunk loop consumes, is m + ln(wa + wb) (reading
    R5). When both sides are empty (lse -inf) the result is (0, -inf), the
    identity element (reading R6)."""
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(la, lb)
    both_empty = ~np.isfinite(m)
    ms = np.where(both_empty, 0.0, m)
    wa = np.where(np.isfinite(la), np.exp(la - ms), 0.0)
    wb = np.where(np.isfinite(lb), np.exp(lb - ms), 0.0)
    den = np.where(both_empty, 1.0, wa + wb)
    out = (wa[..., None] * out_a + wb[..., None] * out_b) / den[..., None]
    lse = np.where(both_empty, NEG_INF, ms + np.log(den))
    out = np.where(both_empty[..., None], 0.0, out)
    return out, lse


# --------------------------------------------------------------------------
# Whole-prefill reference: plain, unchunked, unpaged ([DSMLA] 4.2)
# --------------------------------------------------------------------------

def request_keys_f64(prob, req: int) -> np.ndarray:
    """All latent records a request's new rows may see, in position order:
    its C cached context tokens, then its E new tokens (reading R8: the new
    tokens' latents are a dense bf16 tensor)."""
    C = int(prob.ctx_len[req])
    cu = prob.cu_ext()
    ctx = context_latent_f64(prob, req, 0, C)
    ext = bf16_to_f64(prob.ext_latent[cu[req]:cu[req + 1]])
    return np.concatenate([ctx, ext], axis=0)


def prefill_reference(prob, heads: Optional[Sequence[int]] = None,
                      rows: Optional[dict] = None):
    """Output of two-stage MLA prefill by its plain definition: every new row
    of every request attends, for each head, to all context keys and the
    causal prefix of new keys, in one softmax (no chunks, no paging).

    Returns {req: (out [E_sel, len(heads), 128], lse [E_sel, len(heads)])}.
    ``rows`` maps req -> array of extend-row indices to compute (default all).
    """
    H = prob.H
    heads = list(range(H)) if heads is None else list(heads)
    W = bf16_to_f64(prob.W)
    q_all = prob.q
    cu = prob.cu_ext()
    res = {}
    for r in range(prob.B):
        if rows is not None and r not in rows:
            continue
        C, E = int(prob.ctx_len[r]), int(prob.ext_len[r])
        sel = np.arange(E) if rows is None else np.asarray(rows[r], dtype=np.int64)
        lat = request_keys_f64(prob, r)
        vis = causal_visible(E, C)[sel]
        outs = np.zeros((len(sel), len(heads), D_V))
        lses = np.zeros((len(sel), len(heads)))
        for hi, h in enumerate(heads):
            kn, v = decompress_head(lat[:, :D_C], W, H, h)
            q = bf16_to_f64(q_all[cu[r] + sel, h, :])
            o, l = attend(q, kn, lat[:, D_C:], v, prob.scale, vis)
            outs[:, hi], lses[:, hi] = o, l
        res[r] = (outs, lses)
    return res


def chunked_prefill_f64(prob, chunk: int, heads: Optional[Sequence[int]] = None):
    """The two-stage, chunked prefill ([DSMLA] 4.2 and 4.4) in fp64: for each
    context chunk, gather, decompress through kv_b_proj, attend without mask
    and merge into the running (out, lse); then attend causally over the new
    tokens and merge. Used to pin that chunking plus merging equals the plain
    definition. The first merge starts from the identity (0, -inf)."""
    H = prob.H
    heads = list(range(H)) if heads is None else list(heads)
    W = bf16_to_f64(prob.W)
    cu = prob.cu_ext()
    res = {}
    for r in range(prob.B):
        C, E = int(prob.ctx_len[r]), int(prob.ext_len[r])
        q = bf16_to_f64(prob.q[cu[r]:cu[r + 1]])[:, heads, :]
        acc_o = np.zeros((E, len(heads), D_V))
        acc_l = np.full((E, len(heads)), NEG_INF)
        for s0 in range(0, C, chunk):
            n = min(chunk, C - s0)
            lat = context_latent_f64(prob, r, s0, n)
            for hi, h in enumerate(heads):
                kn, v = decompress_head(lat[:, :D_C], W, H, h)
                o, l = attend(q[:, hi], kn, lat[:, D_C:], v, prob.scale)
                acc_o[:, hi], acc_l[:, hi] = merge_states(acc_o[:, hi], acc_l[:, hi], o, l)
        ext = bf16_to_f64(prob.ext_latent[cu[r]:cu[r + 1]])
        vis = causal_visible(E, 0)
        for hi, h in enumerate(heads):
            kn, v = decompress_head(ext[:, :D_C], W, H, h)
            o, l = attend(q[:, hi], kn, ext[:, D_C:], v, prob.scale, vis)
            acc_o[:, hi], acc_l[:, hi] = merge_states(acc_o[:, hi], acc_l[:, hi], o, l)
        res[r] = (acc_o, acc_l)
    return res


# --------------------------------------------------------------------------
# Absorbed form ([DSMLA] section 3 heading): used only as an identity check
# --------------------------------------------------------------------------

def attend_absorbed(q: np.ndarray, latent: np.ndarray, W: np.ndarray, H: int, h: int,
                    scale: float, visible: Optional[np.ndarray] = None):
    """Same attention with W_UK folded into the query and W_UV applied after:
    q_lat = W_UK^h q_nope (512 wide), s_j = scale (q_lat.c_j + q_rope.k_rope_j),
    out = (sum_j p_j c_j) W_UV^h."""
    Wk = W[:, h * D_NOPE:(h + 1) * D_NOPE]
    Wv = W[:, H * D_NOPE + h * D_V:H * D_NOPE + (h + 1) * D_V]
    q_lat = q[:, :D_NOPE] @ Wk.T                             # [R, 512]
    s = scale * (q_lat @ latent[:, :D_C].T + q[:, D_NOPE:] @ latent[:, D_C:].T)
    if visible is not None:
        s = np.where(visible, s, NEG_INF)
    m = np.max(s, axis=1)
    e = np.exp(s - m[:, None])
    Z = e.sum(axis=1)
    o_lat = (e @ latent[:, :D_C]) / Z[:, None]
    return o_lat @ Wv, m + np.log(Z)


# --------------------------------------------------------------------------
# RoPE and query-side relocation ([REDKNOT] Abstract and section 2)
# --------------------------------------------------------------------------

def rope_angles(pos, dim: int = D_ROPE, base: float = 10000.0) -> np.ndarray:
    """phi[p, k] = pos_p * base^(-2k/dim), k = 0..dim/2-1, in fp64 (reading
    R19: original RoPE frequencies, no YaRN)."""
    k = np.arange(dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * k / dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def rope_rotate(x: np.ndarray, pos, base: float = 10000.0, pairing: str = "interleaved"):
    """Rotate the 64-wide rope vectors x [..., 64] by the angles of position
    pos (broadcast over leading dims). Pair k is (2k, 2k+1) when interleaved,
    (k, k+32) when half-split; y0 = x0 cos - x1 sin, y1 = x0 sin + x1 cos
    (reading R19)."""
    x = np.asarray(x, dtype=np.float64)
    phi = rope_angles(pos, x.shape[-1], base)
    c, s = np.cos(phi), np.sin(phi)
    if pairing == "interleaved":
        x0, x1 = x[..., 0::2], x[..., 1::2]
    else:
        x0, x1 = x[..., :32], x[..., 32:]
    y0 = x0 * c - x1 * s
    y1 = x0 * s + x1 * c
    y = np.empty_like(x)
    if pairing == "interleaved":
        y[..., 0::2], y[..., 1::2] = y0, y1
    else:
        y[..., :32], y[..., 32:] = y0, y1
    return y


def relocate_q(q_rope: np.ndarray, delta: int, base: float = 10000.0,
               pairing: str = "interleaved") -> np.ndarray:
    """Query-side relocation: rotate a query's rope part by -delta so that it
    sits in the canonical frame of a document placed at request offset
    delta ([REDKNOT] section 2, online position restoration)."""
    return rope_rotate(q_rope, -float(delta), base, pairing)


# --------------------------------------------------------------------------
# Local/Global head partition and Equation 4 ([REDKNOT] sections 1-3)
# --------------------------------------------------------------------------

def replace_protected(art_out: np.ndarray, rec_out: np.ndarray, prot_rows: np.ndarray):
    """Local-head outputs: the artifact's rows, with each protected row
    replaced (not added to) by its online recomputation ([REDKNOT] section 2,
    protected rows)."""
    o = np.array(art_out, dtype=np.float64, copy=True)
    o[np.asarray(prot_rows, dtype=np.int64)] = rec_out
    return o


def head_partition_merge(O_L: np.ndarray, O_G: np.ndarray, WaL: np.ndarray,
                         WaG: np.ndarray, Wb: np.ndarray) -> np.ndarray:
    """Equation 4 in its plainest reading ([REDKNOT] sections 1-2): the first
    output projection is sliced by head role, so Local and Global projected
    states add, and the sum goes through the one shared second projection:
    y = (O_L W_aL + O_G W_aG) W_b, with O_L [T, HL*128], O_G [T, HG*128]."""
    T = O_L.shape[0]
    z = O_L.reshape(T, -1) @ WaL + O_G.reshape(T, -1) @ WaG
    return z @ Wb


def _doc_keys_at_request_positions(prob):
    """All documents' keys at their request positions: document d's
    canonical latents with the rope part rotated by +delta_d (direct
    placement), concatenated in document order. Returns (c_kv [N, 512],
    k_rope [N, 64]) in fp64."""
    ckv, kr = [], []
    for d in prob.documents():
        L = int(d["L"])
        lat = bf16_to_f64(gather_bf16_bits(d["pool"], d["block_table"], 0, 0, L))
        ckv.append(lat[:, :D_C])
        kr.append(rope_rotate(lat[:, D_C:], float(d["delta"]), prob.rope_base))
    return np.concatenate(ckv), np.concatenate(kr)


def reuse_reference(prob, global_rows: Optional[np.ndarray] = None):
    """Head-partitioned reuse prefill by definition ([REDKNOT] Abstract,
    sections 2-3; readings R20-R23). Direct placement: each canonical
    document key's rope part is rotated by +delta of its document, which
    puts the document at request positions delta..delta+L-1 where the
    queries' rope parts already are; no query rotation. With several
    documents ([REDKNOT] section 2, segmented merging) the keys of all of
    them, each at its own offset, form one softmax. Global heads attend all
    rows over all keys; Local heads recompute only protected rows; the result
    is Equation 4 over artifact rows with protected rows replaced.

    Returns dict with O_G [T,HG,128], lse_G, rec [P,HL,128], rec_lse, y [T,d_model].
    """
    H, HL = prob.H, prob.n_local
    T = prob.T
    W = bf16_to_f64(prob.W)
    c_kv, k_rope = _doc_keys_at_request_positions(prob)
    q = bf16_to_f64(prob.q)
    prot = np.asarray(prob.prot_rows, dtype=np.int64)
    rows_g = np.arange(T) if global_rows is None else np.asarray(global_rows)
    O_G = np.zeros((len(rows_g), H - HL, D_V))
    l_G = np.zeros((len(rows_g), H - HL))
    for gi, h in enumerate(range(HL, H)):
        kn, v = decompress_head(c_kv, W, H, h)
        O_G[:, gi], l_G[:, gi] = attend(q[rows_g, h], kn, k_rope, v, prob.scale)
    rec = np.zeros((len(prot), HL, D_V))
    rec_l = np.zeros((len(prot), HL))
    for h in range(HL):
        kn, v = decompress_head(c_kv, W, H, h)
        rec[:, h], rec_l[:, h] = attend(q[prot, h], kn, k_rope, v, prob.scale)
    res = dict(O_G=O_G, lse_G=l_G, rec=rec, rec_lse=rec_l)
    if global_rows is None:
        O_L = replace_protected(bf16_to_f64(prob.art_out), rec, prot)
        res["y"] = head_partition_merge(O_L, O_G, bf16_to_f64(prob.WaL),
                                        bf16_to_f64(prob.WaG), bf16_to_f64(prob.Wb))
    return res


def segmented_attention(prob, h: int, rows: np.ndarray):
    """The runtime form of multi-document reuse ([REDKNOT] section 2: online
    relocation rotates queries into each document's canonical frame, attends
    to the canonical latents, and the segment statistics are merged): for
    each document d, q_rope rotated by -delta_d attends to d's canonical keys
    (rope at canonical positions); the per-document (out, lse) are merged
    with merge_states. Equal to the direct placement of reuse_reference by
    RoPE's relative-position property and the merge identity."""
    W = bf16_to_f64(prob.W)
    q = bf16_to_f64(prob.q)[rows, h]
    out = np.zeros((len(rows), D_V))
    lse = np.full(len(rows), NEG_INF)
    for d in prob.documents():
        L = int(d["L"])
        lat = bf16_to_f64(gather_bf16_bits(d["pool"], d["block_table"], 0, 0, L))
        qd = q.copy()
        qd[:, D_NOPE:] = relocate_q(q[:, D_NOPE:], int(d["delta"]), prob.rope_base)
        kn, v = decompress_head(lat[:, :D_C], W, prob.H, h)
        o, l = attend(qd, kn, lat[:, D_C:], v, prob.scale)
        out, lse = merge_states(out, lse, o, l)
    return out, lse


# --------------------------------------------------------------------------
# Offline Local-head artifact ([REDKNOT] Abstract; section 2, "Canonical
# offline artifacts")
# --------------------------------------------------------------------------

def artifact_row_positions(L: int, row_ids, doc_rows: bool) -> np.ndarray:
    """Canonical positions of an artifact's rows (reading R31): with
    doc_rows, rows 0..L-1 are the document's own tokens at positions 0..L-1
    and any further rows follow the document at L, L+1, ... (row i at i);
    without, every row follows the document (row i at L + i)."""
    i = np.asarray(row_ids, dtype=np.int64)
    return i if doc_rows else L + i


def build_artifact(latent: np.ndarray, q: np.ndarray, W: np.ndarray, H: int, n_local: int,
                   scale: float, doc_rows: bool, row_ids=None, heads=None):
    """MLA-Off: the document processed alone at canonical position zero, its
    Local-head results kept ([REDKNOT] Abstract and section 2; reading R31).
    latent [L, 576] (fp64) are the document's records with the rope part at
    canonical positions 0..L-1; q [R, H, 192] (fp64) are the queries of
    artifact rows row_ids (default 0..R-1), rope part at the rows' canonical
    positions (artifact_row_positions). Row r at position p_r sees key t iff
    t <= p_r: a document row attends to itself and the tokens before it, a
    row after the document to all of it. Heads default to the Local heads
    0..n_local-1. Returns (out [R, n_heads, 128], lse [R, n_heads])."""
    L = latent.shape[0]
    R = q.shape[0]
    rows = np.arange(R) if row_ids is None else np.asarray(row_ids, dtype=np.int64)
    hs = list(range(n_local)) if heads is None else list(heads)
    assert all(0 <= h < n_local for h in hs)
    pos = artifact_row_positions(L, rows, doc_rows)
    visible = np.arange(L)[None, :] <= pos[:, None]
    out = np.zeros((R, len(hs), D_V))
    lse = np.zeros((R, len(hs)))
    for j, h in enumerate(hs):
        kn, v = decompress_head(latent[:, :D_C], W, H, h)
        out[:, j], lse[:, j] = attend(q[:, h], kn, latent[:, D_C:], v, scale, visible)
    return out, lse


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a (Fowler-Noll-Vo): start at the offset basis
    14695981039346656037; for each byte, xor it in, then multiply by the
    prime 1099511628211 modulo 2^64."""
    h = 14695981039346656037
    for b in data:
        h = ((h ^ b) * 1099511628211) % (1 << 64)
    return h


def token_bytes(tokens) -> bytes:
    """Token ids as the bytes that are hashed: each id's four little-endian
    bytes (as a 32-bit two's-complement integer), in order."""
    return b"".join((int(t) & 0xFFFFFFFF).to_bytes(4, "little")
                    for t in np.asarray(tokens, dtype=np.int64).tolist())


def artifact_token_hash(tokens) -> int:
    """The token binding of an artifact's description (reading R32):
    fnv1a64 of token_bytes."""
    return fnv1a64(token_bytes(tokens))


ARTIFACT_PROFILE_FIELDS = ("n_heads", "n_local", "d_c", "d_rope", "d_nope", "d_v", "rope_base", "n_layers")


def artifact_check_reason(artifact: dict, request: dict) -> int:
    """Validation before reuse ([REDKNOT] section 2: fall back to full
    recomputation on missing layers, token or profile mismatch, or a stale
    generation; reading R32 fixes the order of the checks as the page lists
    them and leaves out the tensor-parallel and rank checks). Returns 0
    (valid), 1 (a layer the request needs is absent from the artifact's
    layer_mask), 2 (token count or token hash differ), 3 (a profile field
    differs), 4 (generation differs)."""
    if request["layer_mask"] & ~artifact["layer_mask"]:
        return 1
    if artifact["n_tokens"] != request["n_tokens"] or artifact["token_hash"] != request["token_hash"]:
        return 2
    if any(artifact[f] != request[f] for f in ARTIFACT_PROFILE_FIELDS):
        return 3
    if artifact["generation"] != request["generation"]:
        return 4
    return 0


# --------------------------------------------------------------------------
# Layout constants ([DSMLA] 5.2; [PAGED] KV accounting table)
# --------------------------------------------------------------------------

def latent_record_elems(d_c: int = D_C, d_rope: int = D_ROPE) -> int:
    """Elements per cached token per layer: the latent plus the rope key."""
    return d_c + d_rope


def mha_bytes_per_token_layer(heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """Bytes per token per layer of a full per-head K and V cache."""
    return 2 * heads * head_dim * elem_bytes


def fp8_block_bytes(block: int = BLOCK) -> int:
    """Bytes of one fp8 cache block (reading R16): e4m3 c_kv, bf16 k_rope,
    one fp32 scale per token."""
    return block * D_C + block * D_ROPE * 2 + block * 4
