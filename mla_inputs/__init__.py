"""Seeded synthetic inputs for MLA chunked prefill over a paged latent cache.

This module only draws and lays out inputs. It holds none of the method's
arithmetic (no gather, projection, attention, merge or rotation), so the fp64
oracle under ``oracle/`` and the HIP path can both consume its arrays without
sharing any computation.

All floating-point tensors are returned as raw bit patterns:

* bf16 tensors as ``np.uint16`` (upper half of an IEEE fp32, round to nearest
  even from an fp32 draw),
* fp8 tensors as ``np.uint8`` OCP E4M3FN codes,
* fp32 tensors as ``np.float32``.

Cache layouts (one layer):

* bf16 cache: ``pool[num_blocks, 64, 576]`` where each token record is the
  512-wide compressed latent ``c_kv`` followed by the 64-wide ``k_rope``
  (DeepSeek MLA -- Prefix Cache and Chunked Prefill, section 5.2 "MLA KV
  Buffer" layout; 64-token blocks per "PagedAttention assumed MHA",
  section "Block size is not a tuning knob here").
* fp8 cache: ``pool[num_blocks, 41216]`` bytes; per block, structure of
  arrays: ``c_kv`` E4M3FN codes ``[64][512]`` at byte 0, ``k_rope`` bf16
  ``[64][64]`` at byte 32768, per-token fp32 scale ``[64]`` at byte 40960.
  BF16 rope next to FP8 content in one block follows "PagedAttention assumed
  MHA", section "What DeepSeek-V4 breaks".

Draw order for a seed: lengths, block permutation, context latents, extend
latents, q, kv_b_proj, then the head-partitioned-reuse extras (artifact out,
artifact lse, protected rows, W_aL, W_aG, W_b).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

D_C = 512          # compressed latent width
D_ROPE = 64        # shared rope key width
D_LAT = D_C + D_ROPE   # 576 elements per token record
D_NOPE = 128
D_V = 128
D_QK = D_NOPE + D_ROPE  # 192
BLOCK = 64
FP8_MAX = 448.0
FP8_BLOCK_BYTES = BLOCK * D_C + BLOCK * D_ROPE * 2 + BLOCK * 4   # 41216
FP8_ROPE_OFF = BLOCK * D_C                                       # 32768
FP8_SCALE_OFF = FP8_ROPE_OFF + BLOCK * D_ROPE * 2                # 40960
BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even) and return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    return r.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def _normal_bf16_blocks(seed, shape, std: float = 1.0, block: int = 1 << 23) -> np.ndarray:
    """N(0, std^2) bf16 bits for large arrays: the flat array is cut into
    fixed blocks, block i drawn from child i of SeedSequence(seed), so the
    values do not depend on how many threads fill them."""
    import concurrent.futures as cf
    import os
    n = int(np.prod(shape))
    kids = np.random.SeedSequence(seed).spawn(max(1, (n + block - 1) // block))
    out = np.empty(n, dtype=np.uint16)

    def fill(i):
        m = min(block, n - i * block)
        x = np.random.default_rng(kids[i]).standard_normal(size=m, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[i * block:i * block + m] = f32_to_bf16_bits(x)

    with cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(len(kids))))
    return out.reshape(shape)


def _bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_rows_e4m3(x_bf16_bits: np.ndarray):
    """Encode each row of a bf16 matrix as E4M3FN codes with one fp32 scale.

    scale = fp32(max|x|) / 448 (fp32 division), code = e4m3(clamp(x / scale)),
    rounding by torch's float8_e4m3fn cast (round to nearest even). An
    all-zero row gets scale 0 and zero codes. This produces the fp8 cache
    input; dequantisation is not done here.
    """
    import torch

    x = _bf16_bits_to_f32(x_bf16_bits)
    amax = np.max(np.abs(x), axis=-1).astype(np.float32)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)
    y = np.clip(y, -FP8_MAX, FP8_MAX)
    y[scale == 0] = 0.0
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


@dataclasses.dataclass
class Problem:
    """One synthetic MLA prefill problem (a single layer)."""
    name: str
    H: int
    ctx_len: np.ndarray          # int64 [B] cached context tokens per request
    ext_len: np.ndarray          # int64 [B] new (extend) tokens per request
    chunk: int                   # context chunk length in tokens
    cache_dtype: str             # "bf16" or "fp8"
    pool: np.ndarray             # bf16 bits [NB,64,576] or fp8 bytes [NB,41216]
    block_table: np.ndarray      # int32 [B, max_blocks]
    ext_latent: np.ndarray       # bf16 bits [sum E, 576]
    q: np.ndarray                # bf16 bits [T, H, 192] (nope first, rope last)
    W: np.ndarray                # bf16 bits [512, H*256] = [W_UK all heads | W_UV all heads]
    scale: float                 # softmax scale
    seed: int
    # head-partitioned reuse extras (None otherwise)
    delta: Optional[int] = None          # request offset of the document
    rope_base: float = 10000.0
    n_local: int = 0                     # heads [0, n_local) are Local
    art_out: Optional[np.ndarray] = None     # bf16 bits [T, HL, 128]
    art_lse: Optional[np.ndarray] = None     # fp32 [T, HL]
    prot_rows: Optional[np.ndarray] = None   # int32 [P], sorted
    WaL: Optional[np.ndarray] = None         # bf16 bits [HL*128, d_mid]
    WaG: Optional[np.ndarray] = None         # bf16 bits [HG*128, d_mid]
    Wb: Optional[np.ndarray] = None          # bf16 bits [d_mid, d_model]
    # several documents (each its own pool and block table, canonical
    # positions 0..L_d-1, placed at request offset delta_d); None = the one
    # document given by pool / block_table / ctx_len[0] / delta
    docs: Optional[list] = None

    def documents(self) -> list:
        """[dict(pool, block_table, L, delta)] of a reuse problem."""
        if self.docs is not None:
            return self.docs
        return [dict(pool=self.pool, block_table=self.block_table, L=int(self.ctx_len[0]),
                     delta=int(self.delta))]

    @property
    def B(self) -> int:
        return int(self.ctx_len.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.pool.shape[0])

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    def cu_ext(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.ext_len)]).astype(np.int64)

    @property
    def is_reuse(self) -> bool:
        return self.delta is not None


def _build_pool(rng, ctx_len, cache_dtype, extra_blocks=0, poison=False):
    """Draw context latents in logical order and scatter them into a shuffled pool."""
    B = len(ctx_len)
    nblk = [(int(c) + BLOCK - 1) // BLOCK for c in ctx_len]
    used = int(sum(nblk))
    NB = used + int(extra_blocks)
    perm = rng.permutation(NB).astype(np.int32)
    max_nb = max(1, max(nblk))
    bt = np.zeros((B, max_nb), dtype=np.int32)
    off = 0
    for r in range(B):
        bt[r, :nblk[r]] = perm[off:off + nblk[r]]
        off += nblk[r]
    lat = _normal_bf16(rng, (used * BLOCK, D_LAT))          # logical order, whole blocks
    if cache_dtype == "bf16":
        pool = np.empty((NB, BLOCK, D_LAT), dtype=np.uint16)
        if extra_blocks:
            pool[perm[used:]] = BF16_NAN if poison else np.uint16(0)
        pool[perm[:used]] = lat.reshape(used, BLOCK, D_LAT)
    elif cache_dtype == "fp8":
        codes, sc = quantize_rows_e4m3(lat[:, :D_C])
        pool = np.zeros((NB, FP8_BLOCK_BYTES), dtype=np.uint8)
        if extra_blocks and poison:
            pool[perm[used:]] = 0x7F        # E4M3FN NaN codes everywhere
        blk = np.empty((used, FP8_BLOCK_BYTES), dtype=np.uint8)
        blk[:, :FP8_ROPE_OFF] = codes.reshape(used, BLOCK * D_C)
        blk[:, FP8_ROPE_OFF:FP8_SCALE_OFF] = np.ascontiguousarray(
            lat[:, D_C:].reshape(used, BLOCK * D_ROPE)).view(np.uint8)
        blk[:, FP8_SCALE_OFF:] = np.ascontiguousarray(sc.reshape(used, BLOCK)).view(np.uint8)
        pool[perm[:used]] = blk
    else:
        raise ValueError(cache_dtype)
    return pool, bt


def make_problem(H, ctx_len, ext_len, chunk, cache_dtype="bf16", seed=0,
                 extra_blocks=0, poison=False, name="custom", w_std=None,
                 scale=None) -> Problem:
    """A prefill problem with the given per-request lengths.

    Lengths are taken as given (the caller draws them first when they are
    random). Latents and q are N(0,1), kv_b_proj is N(0, 1/512).
    """
    rng = np.random.default_rng(seed)
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    ext_len = np.asarray(ext_len, dtype=np.int64)
    return _finish(rng, name, H, ctx_len, ext_len, chunk, cache_dtype, seed,
                   extra_blocks, poison, w_std, scale)


def _finish(rng, name, H, ctx_len, ext_len, chunk, cache_dtype, seed,
            extra_blocks=0, poison=False, w_std=None, scale=None):
    pool, bt = _build_pool(rng, ctx_len, cache_dtype, extra_blocks, poison)
    T = int(ext_len.sum())
    ext = _normal_bf16(rng, (T, D_LAT))
    q = _normal_bf16(rng, (T, H, D_QK))
    W = _normal_bf16(rng, (D_C, H * (D_NOPE + D_V)), std=(w_std if w_std else 1.0 / np.sqrt(D_C)))
    return Problem(name=name, H=H, ctx_len=ctx_len, ext_len=ext_len, chunk=int(chunk),
                   cache_dtype=cache_dtype, pool=pool, block_table=bt, ext_latent=ext,
                   q=q, W=W, scale=float(scale if scale else 1.0 / np.sqrt(D_QK)), seed=seed)


def make_reuse_problem(H=64, n_local=56, L=262144, T=512, delta=4096, P=64,
                       d_mid=2048, d_model=4096, chunk=8192, seed=5,
                       name="reuse") -> Problem:
    """Head-partitioned reuse: one document at canonical positions 0..L-1,
    T query rows at request positions delta+L+i, Local heads [0, n_local)
    served from a seeded artifact with P protected rows recomputed.

    The artifact is synthetic: out ~ N(0, e/L) (the spread a softmax over L
    N(0,1)-scored keys gives), lse = ln L + 0.5 + 0.1 N(0,1).
    """
    rng = np.random.default_rng(seed)
    ctx_len = np.array([L], dtype=np.int64)
    pool, bt = _build_pool(rng, ctx_len, "bf16")
    q = _normal_bf16(rng, (T, H, D_QK))
    W = _normal_bf16(rng, (D_C, H * (D_NOPE + D_V)), std=1.0 / np.sqrt(D_C))
    HL, HG = n_local, H - n_local
    art_out = _normal_bf16(rng, (T, HL, D_V), std=float(np.sqrt(np.e / max(L, 1))))
    art_lse = (np.log(max(L, 1)) + 0.5 + 0.1 * rng.standard_normal((T, HL))).astype(np.float32)
    prot = np.sort(rng.choice(T, size=P, replace=False)).astype(np.int32)
    WaL = _normal_bf16(rng, (HL * D_V, d_mid), std=1.0 / np.sqrt(HL * D_V))
    WaG = _normal_bf16(rng, (HG * D_V, d_mid), std=1.0 / np.sqrt(HG * D_V))
    Wb = _normal_bf16(rng, (d_mid, d_model), std=1.0 / np.sqrt(d_mid))
    return Problem(name=name, H=H, ctx_len=ctx_len, ext_len=np.array([0], dtype=np.int64),
                   chunk=chunk, cache_dtype="bf16", pool=pool, block_table=bt,
                   ext_latent=np.zeros((0, D_LAT), dtype=np.uint16), q=q, W=W,
                   scale=float(1.0 / np.sqrt(D_QK)), seed=seed, delta=int(delta),
                   n_local=HL, art_out=art_out, art_lse=art_lse, prot_rows=prot,
                   WaL=WaL, WaG=WaG, Wb=Wb)


def make_multidoc_problem(H=8, n_local=7, doc_lens=(512, 192, 1088), T=100, delta=4096, P=7,
                          d_mid=256, d_model=256, chunk=256, seed=6, name="multidoc") -> Problem:
    """Segmented reuse: documents d = 0..n-1, each built at canonical
    positions 0..L_d-1 in a pool of its own, placed one after another in the
    request (document d at offset delta_d = delta + L_0 + ... + L_{d-1});
    T query rows at request positions delta_{n-1} + L_{n-1} + i (their rope
    part is given rotated there). Artifact, protected rows and projections
    as in make_reuse_problem."""
    rng = np.random.default_rng(seed)
    docs = []
    off = int(delta)
    for L in doc_lens:
        pool, bt = _build_pool(rng, np.array([L], dtype=np.int64), "bf16")
        docs.append(dict(pool=pool, block_table=bt, L=int(L), delta=off))
        off += int(L)
    Ltot = int(sum(doc_lens))
    q = _normal_bf16(rng, (T, H, D_QK))
    W = _normal_bf16(rng, (D_C, H * (D_NOPE + D_V)), std=1.0 / np.sqrt(D_C))
    HL, HG = n_local, H - n_local
    art_out = _normal_bf16(rng, (T, HL, D_V), std=float(np.sqrt(np.e / max(Ltot, 1))))
    art_lse = (np.log(max(Ltot, 1)) + 0.5 + 0.1 * rng.standard_normal((T, HL))).astype(np.float32)
    prot = np.sort(rng.choice(T, size=P, replace=False)).astype(np.int32)
    WaL = _normal_bf16(rng, (HL * D_V, d_mid), std=1.0 / np.sqrt(HL * D_V))
    WaG = _normal_bf16(rng, (HG * D_V, d_mid), std=1.0 / np.sqrt(HG * D_V))
    Wb = _normal_bf16(rng, (d_mid, d_model), std=1.0 / np.sqrt(d_mid))
    return Problem(name=name, H=H, ctx_len=np.array([Ltot], dtype=np.int64),
                   ext_len=np.array([0], dtype=np.int64), chunk=chunk, cache_dtype="bf16",
                   pool=docs[0]["pool"], block_table=docs[0]["block_table"],
                   ext_latent=np.zeros((0, D_LAT), dtype=np.uint16), q=q, W=W,
                   scale=float(1.0 / np.sqrt(D_QK)), seed=seed, delta=int(delta),
                   n_local=HL, art_out=art_out, art_lse=art_lse, prot_rows=prot,
                   WaL=WaL, WaG=WaG, Wb=Wb, docs=docs)


@dataclasses.dataclass
class ArtifactProblem:
    """Inputs of an offline Local-head artifact build: one document at
    canonical positions 0..L-1 in a pool of its own, the query rows of the
    artifact with their rope parts at canonical positions (document rows
    first when doc_rows, then rows after the document), kv_b_proj, and the
    document's token ids and content generation for its description."""
    name: str
    H: int
    n_local: int
    L: int
    doc_rows: bool
    pool: np.ndarray             # bf16 bits [NB, 64, 576]
    block_table: np.ndarray      # int32 [1, max_blocks]
    q: np.ndarray                # bf16 bits [R, H, 192]
    W: np.ndarray                # bf16 bits [512, H*256]
    scale: float
    tokens: np.ndarray           # int32 [L] token ids
    generation: int
    seed: int
    chunk: int
    rope_base: float = 10000.0

    @property
    def R(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.pool.shape[0])


def make_artifact_problem(H=8, n_local=7, L=1088, extra_rows=50, doc_rows=True, chunk=256, seed=7,
                          generation=3, vocab=129280, name="artifact") -> ArtifactProblem:
    """A document to build an artifact for: L tokens in a shuffled pool,
    R = (L if doc_rows else 0) + extra_rows query rows (N(0,1), rope part at
    the rows' canonical positions; drawn from SeedSequence([seed, 1]) in
    blocks), kv_b_proj N(0, 1/512), token ids uniform in [0, vocab)."""
    rng = np.random.default_rng(seed)
    pool, bt = _build_pool(rng, np.array([L], dtype=np.int64), "bf16")
    R = (L if doc_rows else 0) + int(extra_rows)
    # the query rows of a long document are large: drawn in parallel blocks
    q = _normal_bf16_blocks([seed, 1], (R, H, D_QK))
    W = _normal_bf16(rng, (D_C, H * (D_NOPE + D_V)), std=1.0 / np.sqrt(D_C))
    tokens = rng.integers(0, vocab, size=L).astype(np.int32)
    return ArtifactProblem(name=name, H=H, n_local=n_local, L=int(L), doc_rows=bool(doc_rows), pool=pool,
                           block_table=bt, q=q, W=W, scale=float(1.0 / np.sqrt(D_QK)), tokens=tokens,
                           generation=int(generation), seed=seed, chunk=int(chunk))


ARTIFACT_CONFIG_NAME = ("MLA-Off artifact build: one 65536-token document at canonical position zero, "
                        "64 heads (56 Local built), every document row causal, one chunk")


def make_artifact_config() -> ArtifactProblem:
    """The offline build measured by the benchmark: the reuse geometry's
    heads (64, Local 0..55), a 65536-token document, every document row."""
    return make_artifact_problem(H=64, n_local=56, L=65536, extra_rows=0, doc_rows=True, chunk=65536, seed=8,
                                 name="artifact")


def document_tokens(L: int, seed: int, vocab: int = 129280) -> np.ndarray:
    """Seeded token ids of a document (int32, uniform in [0, vocab))."""
    return np.random.default_rng(seed).integers(0, vocab, size=L).astype(np.int32)


def ragged_lengths(rng, B=16, ctx_lo=1024, ctx_hi=32768, ext_lo=256, ext_hi=2048):
    """Context lengths uniform in [ctx_lo, ctx_hi] rounded down to a multiple of
    64; extend lengths uniform in [ext_lo, ext_hi] (inclusive)."""
    c = rng.integers(ctx_lo, ctx_hi + 1, size=B)
    c = (c // BLOCK) * BLOCK
    e = rng.integers(ext_lo, ext_hi + 1, size=B)
    return c.astype(np.int64), e.astype(np.int64)


CONFIG_NAMES = {
    1: "tiny: 1 request, 8 heads, 256 ctx (4 of 16 blocks) + 64 new, chunk 128",
    2: "dsv3: 128 heads, 4 requests x (8192 ctx + 1024 new), chunk 4096, bf16",
    3: "long: 128 heads, 1 request x (131072 ctx + 2048 new), chunk 8192, bf16",
    4: "fp8-ragged: 128 heads, 16 requests, ctx U[1024,32768]/64*64, new U[256,2048], chunk 4096",
    5: "reuse: 64 heads (56 Local / 8 Global), 262144-token document, 512 query rows at +4096, chunk 65536",
}


def make_config(k: int) -> Problem:
    """The five standard workloads; seed = config number."""
    if k == 1:
        return make_problem(8, [256], [64], 128, "bf16", seed=1, extra_blocks=12,
                            poison=True, name="tiny")
    if k == 2:
        return make_problem(128, [8192] * 4, [1024] * 4, 4096, "bf16", seed=2, name="dsv3")
    if k == 3:
        return make_problem(128, [131072], [2048], 8192, "bf16", seed=3, name="long")
    if k == 4:
        rng = np.random.default_rng(4)
        c, e = ragged_lengths(rng)
        return _finish(rng, "fp8-ragged", 128, c, e, 4096, "fp8", 4)
    if k == 5:
        # chunk 65536 (the pages fix none for this workload): 4 chunks of
        # 2 GB of decompressed k/v each, large enough to fill the GPU
        return make_reuse_problem(chunk=65536, seed=5, name="reuse")
    raise ValueError(k)
