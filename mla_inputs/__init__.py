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
    """Round fp32 values to bf16 (nearest even) and return the bit patterns.

    Large arrays are converted in cache-sized pieces on several threads (the
    result does not depend on the split)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).reshape(-1)
    out = np.empty(u.shape, dtype=np.uint16)
    piece = 1 << 20

    def conv(s):
        t = u[s:s + piece]
        r = t >> np.uint32(16)
        r &= np.uint32(1)
        r += np.uint32(0x7FFF)
        r += t
        r >>= np.uint32(16)
        out[s:s + piece] = r

    starts = range(0, u.size, piece)
    if u.size > 4 * piece:
        import concurrent.futures as cf
        import os
        with cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
            list(ex.map(conv, starts))
    else:
        for s in starts:
            conv(s)
    return out.reshape(x.shape)


_BIG = 1 << 24      # arrays above this many elements are drawn in parallel blocks


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws rounded to bf16. Arrays of more than 2^24 elements
    take one 64-bit seed from rng and are drawn in parallel blocks from it
    (_normal_bf16_blocks), so that the largest workloads' inputs are ready
    in seconds; smaller ones are drawn from rng directly."""
    if int(np.prod(shape)) > _BIG:
        return _normal_bf16_blocks(int(rng.integers(0, 2 ** 63, dtype=np.int64)), shape, std)
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
    input; dequantisation is not done here. (torch's CPU ops, which divide
    with IEEE fp32 rounding, do the elementwise work on several threads.)
    """
    import torch

    xb = torch.from_numpy(np.ascontiguousarray(x_bf16_bits).view(np.int16)).view(torch.bfloat16)
    x = xb.to(torch.float32)
    amax = x.abs().amax(dim=-1)
    scale = amax / torch.tensor(FP8_MAX, dtype=torch.float32)
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    y = (x / safe.unsqueeze(-1)).clamp_(-FP8_MAX, FP8_MAX)
    y[scale == 0] = 0.0
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale.numpy()


def selection_kv_b_proj(rng: np.random.Generator, H: int) -> np.ndarray:
    """A kv_b_proj [512, H*256] (bf16 bits) whose every column picks one
    latent dimension with weight +-1/4 or +-1/8: the 128 key columns of a
    head pick distinct dimensions, and so do its 128 value columns. Every
    k_nope and v entry it produces is then a latent entry times a power of
    two, so it is exactly representable in bf16 whatever the arithmetic
    order, and the absorbed query W_UK q_nope has at most one term per latent
    dimension. Edge-case problems use it so that rounding of decompressed
    keys cannot mask a wrong key set (a dropped or duplicated key moves the
    lse of an n-key row by about 1/n). The small weights keep values and
    outputs of a softmax over a few keys near the size they have over many
    (a fraction of one), where the absolute output bar is a few bf16 ulps."""
    W = np.zeros((D_C, H * (D_NOPE + D_V)), dtype=np.float32)
    vals = np.array([-0.25, -0.125, 0.125, 0.25], dtype=np.float32)
    for blk in range(2 * H):      # blocks 0..H-1: W_UK of head blk; H..2H-1: W_UV of head blk-H
        rows = rng.choice(D_C, size=D_NOPE, replace=False)
        W[rows, blk * D_NOPE + np.arange(D_NOPE)] = vals[rng.integers(0, 4, size=D_NOPE)]
    return f32_to_bf16_bits(W)


def _kv_b_proj(rng, H, weights="normal", w_std=None):
    if weights == "selection":
        return selection_kv_b_proj(rng, H)
    if weights != "normal":
        raise ValueError(weights)
    return _normal_bf16(rng, (D_C, H * (D_NOPE + D_V)), std=(w_std if w_std else 1.0 / np.sqrt(D_C)))


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


def _build_pool(rng, ctx_len, cache_dtype, extra_blocks=0, poison=False, exact_dequant=False):
    """Draw context latents in logical order and scatter them into a shuffled pool.

    exact_dequant (fp8 only): every record's c_kv gets its largest magnitude
    at exactly 7 = 448 / 64 (values clipped to [-6.5, 6.5], one seeded
    position per record set to +-7), so its scale is 2^-6 and every
    dequantised value (code times 2^-6) is exactly representable in bf16."""
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
    if exact_dequant:
        if cache_dtype != "fp8":
            raise ValueError("exact_dequant applies to the fp8 cache")
        x = np.clip(_bf16_bits_to_f32(lat[:, :D_C]), -6.5, 6.5)
        pos = rng.integers(0, D_C, size=x.shape[0])
        sgn = np.where(rng.integers(0, 2, size=x.shape[0]) == 1, 7.0, -7.0).astype(np.float32)
        x[np.arange(x.shape[0]), pos] = sgn
        lat = lat.copy()
        lat[:, :D_C] = f32_to_bf16_bits(x)
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
                 scale=None, weights="normal", exact_dequant=False) -> Problem:
    """A prefill problem with the given per-request lengths.

    Lengths are taken as given (the caller draws them first when they are
    random). Latents and q are N(0,1), kv_b_proj is N(0, 1/512)
    (weights="normal") or a selection matrix (weights="selection",
    selection_kv_b_proj); exact_dequant as in _build_pool.
    """
    rng = np.random.default_rng(seed)
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    ext_len = np.asarray(ext_len, dtype=np.int64)
    return _finish(rng, name, H, ctx_len, ext_len, chunk, cache_dtype, seed,
                   extra_blocks, poison, w_std, scale, weights, exact_dequant)


def _finish(rng, name, H, ctx_len, ext_len, chunk, cache_dtype, seed,
            extra_blocks=0, poison=False, w_std=None, scale=None, weights="normal",
            exact_dequant=False):
    pool, bt = _build_pool(rng, ctx_len, cache_dtype, extra_blocks, poison, exact_dequant)
    T = int(ext_len.sum())
    ext = _normal_bf16(rng, (T, D_LAT))
    q = _normal_bf16(rng, (T, H, D_QK))
    W = _kv_b_proj(rng, H, weights, w_std)
    return Problem(name=name, H=H, ctx_len=ctx_len, ext_len=ext_len, chunk=int(chunk),
                   cache_dtype=cache_dtype, pool=pool, block_table=bt, ext_latent=ext,
                   q=q, W=W, scale=float(scale if scale else 1.0 / np.sqrt(D_QK)), seed=seed)


def _synthetic_artifact(rng, T, HL, L):
    """Seeded Local-head artifact rows for a document of L keys: out ~
    N(0, e/L), lse = ln L + 0.5 + 0.1 N(0,1); for L = 0 the draws are made
    (so later draws do not move) and replaced by the empty state (0, -inf)."""
    art_out = _normal_bf16(rng, (T, HL, D_V), std=float(np.sqrt(np.e / max(L, 1))))
    art_lse = (np.log(max(L, 1)) + 0.5 + 0.1 * rng.standard_normal((T, HL))).astype(np.float32)
    if L == 0:
        art_out[:] = 0
        art_lse[:] = -np.inf
    return art_out, art_lse


def make_reuse_problem(H=64, n_local=56, L=262144, T=512, delta=4096, P=64,
                       d_mid=2048, d_model=4096, chunk=8192, seed=5,
                       name="reuse", weights="normal") -> Problem:
    """Head-partitioned reuse: one document at canonical positions 0..L-1,
    T query rows at request positions delta+L+i, Local heads [0, n_local)
    served from a seeded artifact with P protected rows recomputed.

    The artifact is synthetic: out ~ N(0, e/L) (the spread a softmax over L
    N(0,1)-scored keys gives), lse = ln L + 0.5 + 0.1 N(0,1). An empty
    document's artifact is the empty state, out = 0 and lse = -inf (what the
    offline build writes for it).
    """
    rng = np.random.default_rng(seed)
    ctx_len = np.array([L], dtype=np.int64)
    pool, bt = _build_pool(rng, ctx_len, "bf16")
    q = _normal_bf16(rng, (T, H, D_QK))
    W = _kv_b_proj(rng, H, weights)
    HL, HG = n_local, H - n_local
    art_out, art_lse = _synthetic_artifact(rng, T, HL, L)
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
                          d_mid=256, d_model=256, chunk=256, seed=6, name="multidoc",
                          weights="normal") -> Problem:
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
    W = _kv_b_proj(rng, H, weights)
    HL, HG = n_local, H - n_local
    art_out, art_lse = _synthetic_artifact(rng, T, HL, Ltot)
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
                          generation=3, vocab=129280, name="artifact", weights="normal") -> ArtifactProblem:
    """A document to build an artifact for: L tokens in a shuffled pool,
    R = (L if doc_rows else 0) + extra_rows query rows (N(0,1), rope part at
    the rows' canonical positions; drawn from SeedSequence([seed, 1]) in
    blocks), kv_b_proj N(0, 1/512), token ids uniform in [0, vocab)."""
    rng = np.random.default_rng(seed)
    pool, bt = _build_pool(rng, np.array([L], dtype=np.int64), "bf16")
    R = (L if doc_rows else 0) + int(extra_rows)
    # the query rows of a long document are large: drawn in parallel blocks
    q = _normal_bf16_blocks([seed, 1], (R, H, D_QK))
    W = _kv_b_proj(rng, H, weights)
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
