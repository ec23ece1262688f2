"""Host orchestration of MLA prefill over the C ABI (argument marshalling and
launch order only; every step runs in the HIP kernels of libmla.so).

ChunkedPrefill -- the two-stage prefill of "DeepSeek MLA -- Prefix Cache and
Chunked Prefill" (section 4.2) with the context-chunk loop of section 4.4:
for each context chunk: gather -> decompress -> attention (no mask) -> merge;
then the new tokens: decompress -> causal attention -> merge into the final
(out, lse).

ReusePrefill -- head-partitioned reuse of RedKnot-MLA (Abstract, sections
1-3): queries are relocated into the document's canonical frame, Global heads
are recomputed over the whole document for every row, Local heads only for
the protected rows; Local rows come from the artifact with protected rows
replaced, and the sliced first projection plus the shared second projection
give the layer output (Equation 4).

ArtifactBuilder -- the offline step before that reuse (RedKnot-MLA Abstract
and section 2, "Canonical offline artifacts"): one document processed alone
at canonical position zero, Local heads only, its (out, lse) kept with a
description (tokens, profile, generation, layers) that the reuse path checks
with mla_artifact_check before it trusts the artifact; on any mismatch it
recomputes the Local heads for every row instead.

PyTorch provides device memory and the stream; nothing here computes.
"""
from __future__ import annotations

import contextlib

import numpy as np
import torch

from . import _lib as L

D_LAT = 576
D_V = 128
D_QK = 192


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def _i32(a, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(device)


def _cu(lens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


_NULL = contextlib.nullcontext()


def _span(timer, name):
    """Timing span around one launch when a timer (bench.py) is given."""
    return _NULL if timer is None else timer.span(name)


def pack_weight(w_bits: np.ndarray, device, stream=None) -> torch.Tensor:
    """Upload a bf16 [K][N] weight and store it as [N][K] with mla_pack_weight_t."""
    w = _bf16(w_bits, device)
    K, N = w.shape
    wt = torch.empty((N, K), dtype=torch.bfloat16, device=device)
    L.mla_pack_weight_t(w, K, N, wt, stream)
    return wt


def upload_pool(prob, device) -> torch.Tensor:
    if prob.cache_dtype == "bf16":
        return _bf16(prob.pool, device)
    return torch.from_numpy(np.ascontiguousarray(prob.pool)).to(device)


def _capturing() -> bool:
    return torch.cuda.is_available() and torch.cuda.is_current_stream_capturing()


class _DeviceStatus:
    """The device status word every gather of a driver reports into (a block
    id outside the pool makes the gather write zeros for those tokens and
    store MLA_ERR_OUT_OF_RANGE there)."""

    def check(self, stream=None):
        """Wait for the work enqueued so far, then raise MlaError if a kernel
        stored an error in the status word; the word is cleared for the next
        step either way. Not allowed while a graph is being captured."""
        if stream is None:
            torch.cuda.synchronize(self.dev_status.device)
        else:
            stream.synchronize()
        code = int(self.dev_status.item())
        if code != 0:
            self.dev_status.zero_()
            L.raise_on_device_status(code, type(self).__name__)

    def _finish(self, check, stream):
        if check and not _capturing():
            self.check(stream)


class ChunkedPrefill(_DeviceStatus):
    """Configs with a paged context and new (extend) tokens per request."""

    def __init__(self, prob, device="cuda", chunk=None, fuse_merge="all", two_segment=True, fp8_mode="raw",
                 fold_causal=True, gather_all=None):
        """fp8_mode (fp8 caches): "raw" gathers the codes and scales as they
        are and the decompression reads the codes (mla_gather_context_fp8_raw,
        mla_decompress with row_scale); "dequant" has the gather write the
        dequantised bf16 latent instead.

        With every merge fused and two_segment, each request's causal pass
        over its new tokens runs in the pass of its own last context chunk
        (fold_causal, mla_prefill_attn_chunk); fold_causal=False runs all of
        them in the pass of the loop's last chunk (mla_prefill_attn_2seg).

        gather_all: gather every chunk's records in one launch at the start
        of a step (None: whenever the chunks times the requests fit one
        launch's grid), or each chunk's before its decompression (False)."""
        self.prob = prob
        self.device = device
        assert fuse_merge in ("none", "final", "all")
        assert fp8_mode in ("raw", "dequant")
        self.fuse_merge = fuse_merge
        H = self.H = prob.H
        self.B = prob.B
        self.S = int(chunk or prob.chunk)
        self.cache_dtype = L.DTYPE_BF16 if prob.cache_dtype == "bf16" else L.DTYPE_FP8_E4M3
        self.fp8_raw = prob.cache_dtype == "fp8" and fp8_mode == "raw"
        self.pool = upload_pool(prob, device)
        self.bt = _i32(prob.block_table, device)
        self.ext = _bf16(prob.ext_latent, device)
        self.q = _bf16(prob.q, device)
        self.w_t = pack_weight(prob.W, device)
        self.T = int(prob.ext_len.sum())
        self.maxE = int(prob.ext_len.max()) if self.B else 0
        self.cu_ext = _i32(_cu(prob.ext_len), device)
        # chunk plan: chunk c of request r covers context tokens [c*S, min((c+1)*S, C_r))
        C = prob.ctx_len.astype(np.int64)
        n_chunks = int(max((int(c) + self.S - 1) // self.S for c in C)) if self.B else 0
        self.chunks = []
        off = 0
        starts, lens = [], []
        for c in range(n_chunks):
            start = np.full(self.B, c * self.S, dtype=np.int64)
            ln = np.clip(C - c * self.S, 0, self.S)
            self.chunks.append(dict(start=_i32(start, device), len=_i32(ln, device),
                                    cu=_i32(_cu(ln), device), n=int(ln.sum()), max_len=int(ln.max()),
                                    lat_off=off))
            starts.append(start)
            lens.append(ln)
            off += int(ln.sum())
        max_ctx_tok = max([ch["n"] for ch in self.chunks] + [1])
        # Every chunk's records are gathered by one launch at the start of a
        # step, into one workspace where chunk c's records start at row
        # lat_off: each (chunk, request) is a request of that launch, with
        # the request's block-table row repeated per chunk.
        self.gather_once = bool(self.chunks) and n_chunks * self.B <= 65535 and gather_all is not False
        if self.gather_once:
            self.g_start = _i32(np.concatenate(starts), device)
            self.g_len = _i32(np.concatenate(lens), device)
            self.g_cu = _i32(_cu(np.concatenate(lens)), device)
            self.g_bt = _i32(np.tile(prob.block_table, (n_chunks, 1)), device)
            self.g_batch = n_chunks * self.B
            self.g_max = max(int(np.concatenate(lens).max()), 0)
        else:
            for ch in self.chunks:
                ch["lat_off"] = 0
        # With every merge fused, the last chunk's pass also covers the new
        # tokens (mla_prefill_attn_2seg): their keys are decompressed behind
        # the chunk's, at token offset ext_off of the same workspaces.
        self.two_seg = two_segment and fuse_merge == "all" and bool(self.chunks)
        # fold: request r's new tokens join the pass of its last chunk
        # max(ceil(C_r / S) - 1, 0); last[c][r] marks it
        self.fold = self.two_seg and fold_causal
        if self.fold:
            last_c = np.maximum((C + self.S - 1) // self.S - 1, 0)
            self.last_flags = [_i32((last_c == c).astype(np.int32), device) for c in range(n_chunks)]
        self.ext_off = max_ctx_tok if self.two_seg else 0
        self.max_tok = max([ch["n"] for ch in self.chunks] + [self.ext_off + self.T, 1])
        lat_rows = max(off, 1) if self.gather_once else max_ctx_tok
        self.lat_ws = torch.empty((lat_rows, D_LAT), dtype=torch.bfloat16, device=device)
        # raw fp8 records: codes in the rows' first 512 bytes, scales here
        self.scale_ws = torch.empty(lat_rows, dtype=torch.float32, device=device) if self.fp8_raw else None
        self.k_ws = torch.empty((H, self.max_tok, D_V), dtype=torch.bfloat16, device=device)
        self.v_ws = torch.empty((H, self.max_tok, D_V), dtype=torch.bfloat16, device=device)
        self.hstride = self.max_tok * D_V
        T = max(self.T, 1)
        self.acc_o = torch.empty((T, H, D_V), dtype=torch.float32, device=device)
        self.acc_l = torch.empty((T, H), dtype=torch.float32, device=device)
        if fuse_merge != "all":
            self.tmp_o = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=device)
            self.tmp_l = torch.empty((T, H), dtype=torch.float32, device=device)
        self.out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=device)
        # folded passes write each request's final lse over its state's
        self.lse = self.acc_l if self.fold else torch.empty((T, H), dtype=torch.float32, device=device)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=device)

    # one step of the path per call
    def _gather(self, bt, start, ln, cu, batch, max_len, stream):
        if self.fp8_raw:
            L.mla_gather_context_fp8_raw(self.pool, self.prob.num_blocks, bt, bt.shape[1], start, ln, cu, batch,
                                         max_len, self.lat_ws, self.scale_ws, self.dev_status, stream)
        else:
            L.mla_gather_context(self.pool, self.cache_dtype, self.prob.num_blocks, bt, bt.shape[1], start, ln,
                                 cu, batch, max_len, self.lat_ws, self.dev_status, stream)

    def gather(self, ch, stream=None):
        """The records of chunk ch (when they are not gathered all at once)."""
        self._gather(self.bt, ch["start"], ch["len"], ch["cu"], self.B, ch["max_len"], stream)

    def gather_all(self, stream=None):
        """Every chunk's records in one launch (chunk c's from row lat_off)."""
        self._gather(self.g_bt, self.g_start, self.g_len, self.g_cu, self.g_batch, self.g_max, stream)

    def _lat(self, ch):
        # device address of chunk ch's first record in the latent workspace
        return self.lat_ws.data_ptr() + ch["lat_off"] * D_LAT * 2

    def _scale(self, ch):
        # device address of chunk ch's first scale (raw fp8 records), or None
        return None if not self.fp8_raw else self.scale_ws.data_ptr() + ch["lat_off"] * 4

    def decompress(self, latent, n, stream=None, off=0, row_scale=None):
        """k_nope / v of n tokens into the workspaces from token `off` on
        (row_scale: the rows hold fp8 codes, see mla_decompress)."""
        L.mla_decompress(latent, D_LAT, row_scale, n, self.w_t, self.H, 0, self.H, self._at(self.k_ws, off),
                         self.hstride, self._at(self.v_ws, off), self.hstride, stream)

    @staticmethod
    def _at(ws, off):
        # device address of token `off` of head 0 in a [H, tokens, 128] bf16 workspace
        return ws.data_ptr() + off * D_V * 2

    def attend_2seg(self, ch, merge, stream=None):
        """The last chunk's keys (all visible) and the new tokens' keys
        (causal) in one pass, merged into the running state when `merge`;
        writes the bf16 result."""
        L.mla_prefill_attn_2seg(self.q, self.H * D_QK, self.H, 0, self.H, self.k_ws, self.hstride,
                                self.v_ws, self.hstride, self._lat(ch), D_LAT, ch["cu"],
                                self._at(self.k_ws, self.ext_off), self.hstride,
                                self._at(self.v_ws, self.ext_off), self.hstride, self.ext, D_LAT,
                                self.cu_ext, self.cu_ext, self.B, self.maxE, self.prob.scale,
                                self.acc_o if merge else None, self.H * D_V,
                                self.acc_l if merge else None, self.H, self.out, L.DTYPE_BF16,
                                self.H * D_V, self.lse, self.H, stream)

    def attend_chunk(self, ci, ch, stream=None):
        """Chunk ci's keys for every request, plus the new tokens' keys
        (causal) of the requests whose last chunk this is; those rows get
        their bf16 result, the others' running fp32 state is written (the
        first chunk) or merged into (the chunks after it)."""
        L.mla_prefill_attn_chunk(self.q, self.H * D_QK, self.H, 0, self.H, self.k_ws, self.hstride,
                                 self.v_ws, self.hstride, self._lat(ch), D_LAT, ch["cu"],
                                 self._at(self.k_ws, self.ext_off), self.hstride,
                                 self._at(self.v_ws, self.ext_off), self.hstride, self.ext, D_LAT,
                                 self.cu_ext, self.last_flags[ci], self.cu_ext, self.B, self.maxE,
                                 self.prob.scale, ci > 0, self.acc_o, self.H * D_V, self.acc_l, self.H,
                                 self.out, self.H * D_V, stream)

    def attend(self, latent, cu_k, causal, out, out_dtype, lse, stream=None):
        L.mla_prefill_attn(self.q, self.H * D_QK, self.H, 0, self.H, self.k_ws, self.hstride,
                           self.v_ws, self.hstride, latent, D_LAT, self.cu_ext, cu_k, None, self.B,
                           self.maxE, self.prob.scale, causal, out, out_dtype, self.H * D_V, lse,
                           self.H, stream)

    def attend_merge(self, latent, cu_k, causal, out, out_dtype, lse, stream=None):
        """Attention merged into the running fp32 state (acc_o, acc_l)."""
        L.mla_prefill_attn_merge(self.q, self.H * D_QK, self.H, 0, self.H, self.k_ws, self.hstride,
                                 self.v_ws, self.hstride, latent, D_LAT, self.cu_ext, cu_k, None,
                                 self.B, self.maxE, self.prob.scale, causal, self.acc_o, self.H * D_V,
                                 self.acc_l, self.H, out, out_dtype, self.H * D_V, lse, self.H, stream)

    def merge(self, a, da, la, b, db, lb, out, dout, lout, stream=None):
        L.mla_merge_states(a, da, la, b, db, lb, self.T * self.H, out, dout, lout, stream)

    def run(self, stream=None, timer=None, check=True):
        """One pass of the chunk loop. Chunk 0's attention writes the running
        fp32 state (acc). Each later chunk, and then the causal pass over the
        new tokens, is merged into it, either by mla_merge_states after the
        attention wrote a bf16 chunk state, or inside the attention kernel
        (mla_prefill_attn_merge): fuse_merge selects which merges are fused
        ("none", "final" = only the last, "all"). The last merge writes the
        bf16 result. With "all", the causal pass shares a launch with a
        context chunk: by default each request's with the pass of its own
        last chunk (mla_prefill_attn_chunk), with fold_causal=False all of
        them with the pass of the loop's last chunk (mla_prefill_attn_2seg).

        check: wait for the step and raise if the gather met a block id
        outside the pool (skipped under graph capture; a caller timing steps
        passes False and calls check() afterwards)."""
        out = self._run(stream, timer)
        self._finish(check, stream)
        return out

    def _run(self, stream, timer):
        if self.T == 0:
            return self.out, self.lse
        fuse_mid = self.fuse_merge == "all"
        fuse_last = self.fuse_merge in ("all", "final")
        if self.gather_once:
            with _span(timer, "gather"):
                self.gather_all(stream)
        if self.fold:
            # the new tokens' keys first: every chunk's pass may take some
            with _span(timer, "decompress"):
                self.decompress(self.ext, self.T, stream, off=self.ext_off)
            for ci, ch in enumerate(self.chunks):
                if not self.gather_once:
                    with _span(timer, "gather"):
                        self.gather(ch, stream)
                with _span(timer, "decompress"):
                    self.decompress(self._lat(ch), ch["n"], stream, row_scale=self._scale(ch))
                with _span(timer, "attn_ctx" if ci == 0 else "attn_ctx_merge"):
                    self.attend_chunk(ci, ch, stream)
            return self.out, self.lse
        for ci, ch in enumerate(self.chunks):
            if not self.gather_once:
                with _span(timer, "gather"):
                    self.gather(ch, stream)
            lat = self._lat(ch)
            with _span(timer, "decompress"):
                self.decompress(lat, ch["n"], stream, row_scale=self._scale(ch))
            if self.two_seg and ci == len(self.chunks) - 1:
                with _span(timer, "decompress"):
                    self.decompress(self.ext, self.T, stream, off=self.ext_off)
                with _span(timer, "attn_last"):
                    self.attend_2seg(ch, ci > 0, stream)
                return self.out, self.lse
            if ci == 0:
                with _span(timer, "attn_ctx"):
                    self.attend(lat, ch["cu"], 0, self.acc_o, L.DTYPE_FP32, self.acc_l, stream)
            elif fuse_mid:
                with _span(timer, "attn_ctx_merge"):
                    self.attend_merge(lat, ch["cu"], 0, self.acc_o, L.DTYPE_FP32, self.acc_l, stream)
            else:
                with _span(timer, "attn_ctx"):
                    self.attend(lat, ch["cu"], 0, self.tmp_o, L.DTYPE_BF16, self.tmp_l, stream)
                with _span(timer, "merge"):
                    self.merge(self.acc_o, L.DTYPE_FP32, self.acc_l, self.tmp_o, L.DTYPE_BF16,
                               self.tmp_l, self.acc_o, L.DTYPE_FP32, self.acc_l, stream)
        with _span(timer, "decompress"):
            self.decompress(self.ext, self.T, stream)
        if not self.chunks:
            with _span(timer, "attn_ext"):
                self.attend(self.ext, self.cu_ext, 1, self.out, L.DTYPE_BF16, self.lse, stream)
        elif fuse_last:
            with _span(timer, "attn_ext"):
                self.attend_merge(self.ext, self.cu_ext, 1, self.out, L.DTYPE_BF16, self.lse, stream)
        else:
            with _span(timer, "attn_ext"):
                self.attend(self.ext, self.cu_ext, 1, self.tmp_o, L.DTYPE_BF16, self.tmp_l, stream)
            with _span(timer, "merge"):
                self.merge(self.acc_o, L.DTYPE_FP32, self.acc_l, self.tmp_o, L.DTYPE_BF16, self.tmp_l,
                           self.out, L.DTYPE_BF16, self.lse, stream)
        return self.out, self.lse

    # ---------------------------------------------------------------- accounting
    def work(self) -> dict:
        """Algorithmic work of one run: 2*512*256 flop per decompressed
        (token, head); 640 flop per visible (row, key, head); bytes for the
        HBM-bound steps (gather 2304 B/token bf16, 1796 B/token fp8; merge
        per (row, head) = reads + writes of both states)."""
        p, H = self.prob, self.H
        C = p.ctx_len.astype(np.int64)
        E = p.ext_len.astype(np.int64)
        dec_tok = int(C.sum() + E.sum())
        ctx_pairs = int((C * E).sum())
        ext_pairs = int((E * (E + 1) // 2).sum())
        # context pairs per chunk: chunk 0's plain pass, the merging passes
        # of the chunks after it, and the last chunk (whose pass also takes
        # the new tokens when the chunk loop ends in one two-segment launch)
        pairs = [int((np.clip(C - c * self.S, 0, self.S) * E).sum()) for c in range(len(self.chunks))]
        if getattr(self, "fold", False):
            # each request's causal pairs belong to the pass of its last chunk
            last_c = np.maximum((C + self.S - 1) // self.S - 1, 0)
            passes = [p + int((E * (E + 1) // 2)[last_c == c].sum()) for c, p in enumerate(pairs)]
            return dict(
                dec_flops=2 * 512 * 256 * H * dec_tok,
                attn_flops=640 * H * (ctx_pairs + ext_pairs),
                ctx_attn_flops=640 * H * passes[0],
                ctx_merge_attn_flops=640 * H * sum(passes[1:]),
                ext_attn_flops=0, last_attn_flops=0,
                gather_tokens=int(C.sum()),
                gather_bytes=int(C.sum()) * (2304 if p.cache_dtype == "bf16" else 644 + (644 if self.fp8_raw else 1152)),
                new_tokens=int(E.sum()), ctx_tokens=int(C.sum()), merges=max(len(self.chunks) - 1, 0),
            )
        last_pairs = pairs[-1] if pairs else 0
        first_pairs = pairs[0] if pairs and not (self.two_seg and len(pairs) == 1) else 0
        mid_pairs = ctx_pairs - first_pairs - (last_pairs if self.two_seg else 0)
        n_merge = max(len(self.chunks) - 1, 0) + (1 if self.chunks else 0)
        return dict(
            dec_flops=2 * 512 * 256 * H * dec_tok,
            attn_flops=640 * H * (ctx_pairs + ext_pairs),
            ctx_attn_flops=640 * H * first_pairs,
            ctx_merge_attn_flops=640 * H * mid_pairs,
            ext_attn_flops=0 if self.two_seg else 640 * H * ext_pairs,
            last_attn_flops=640 * H * (last_pairs + ext_pairs) if self.two_seg else 0,
            gather_tokens=int(C.sum()),
            gather_bytes=int(C.sum()) * (2304 if p.cache_dtype == "bf16" else 644 + (644 if self.fp8_raw else 1152)),
            new_tokens=int(E.sum()), ctx_tokens=int(C.sum()), merges=n_merge,
        )


class ReusePrefill(_DeviceStatus):
    """Head-partitioned reuse over one or more documents stored at canonical
    positions. Each document is visited in turn: the queries are relocated by
    its request offset (and re-absorbed for the Local rows), then its chunks
    run as below; the pieces of all documents join one merge tree.

    Local heads (protected rows only) take the absorbed form by default
    (local_path="absorbed"): W_UK is folded into their queries and they
    attend to the gathered latent directly, so only the Global heads are
    decompressed; local_path="decompressed" decompresses every head instead.

    Per document chunk: gather, decompression of the heads that need it, then attention
    of the Global heads (all query rows) and of the Local heads (protected
    rows only). There are few query rows, so one (head, row tile) per
    workgroup would leave most of the GPU idle: every chunk's keys are split
    into `split`-key pieces, each passed to mla_prefill_attn as a request of
    its own (the query rows repeated through q_row_ids), and the partial
    (out, lse) states of all pieces are merged at the end, in one pass over
    them (mla_merge_states_sets; merge="tree" uses a log-depth tree of
    mla_merge_states calls instead). By the merge identity this equals the
    chunk-by-chunk merge."""

    def __init__(self, prob, device="cuda", chunk=None, split=4096, local_path="absorbed",
                 split_local=None, artifact=None, request=None, merge="one_pass"):
        assert prob.is_reuse
        assert local_path in ("absorbed", "decompressed")
        assert merge in ("one_pass", "tree")
        self.merge_mode = merge
        self.prob = prob
        prot_rows = np.asarray(prob.prot_rows, dtype=np.int64)
        # An artifact built offline (ArtifactBuilder) replaces the problem's
        # Local-head rows once its description passes the check against what
        # the request needs; otherwise the Local heads are recomputed for
        # every row (all rows protected, every head decompressed) and the
        # artifact is never read. The decision precedes every launch.
        self.fallback = None
        if artifact is not None:
            if request is None:
                raise ValueError("ReusePrefill: an artifact needs the request's description to be checked against")
            reason = L.mla_artifact_check(artifact.meta, request)
            if reason != L.ARTIFACT_VALID:
                self.fallback = L.ARTIFACT_REASONS[reason]
            elif tuple(artifact.out.shape) != (prob.T, prob.n_local, D_V):
                raise ValueError(f"ReusePrefill: artifact rows {tuple(artifact.out.shape)} do not match "
                                 f"({prob.T}, {prob.n_local}, {D_V})")
        if self.fallback is not None:
            prot_rows = np.arange(prob.T, dtype=np.int64)
            local_path = "decompressed"
        if len(prot_rows) and (np.any(np.diff(prot_rows) <= 0) or prot_rows[0] < 0 or prot_rows[-1] >= prob.T):
            raise ValueError("ReusePrefill: protected rows must be strictly increasing row indices below T")
        self.device = device
        self.local_path = local_path
        self.absorbed = local_path == "absorbed"
        H = self.H = prob.H
        self.HL, self.HG = prob.n_local, H - prob.n_local
        self.S = int(chunk or prob.chunk)
        self.split = max(64, int(split) // 64 * 64)
        # The absorbed Local rows take 128 (row, head) pairs per workgroup and
        # one workgroup per compute unit (its LDS ring fills most of a CU).
        # By default a chunk is cut into as many pieces as fill the GPU in one
        # round with its row tiles, floor(CUs / row tiles), of at least 2048
        # keys each; split_local (keys per piece) overrides.
        if local_path == "absorbed":
            if split_local is None:
                n_rt = -(-(len(prot_rows) * prob.n_local) // 128)
                cus = torch.cuda.get_device_properties(torch.device(device)).multi_processor_count
                per_chunk = max(1, cus // max(n_rt, 1))
                keys = (self.S + per_chunk - 1) // per_chunk            # keys per piece, rounded up
                split_local = max(2048, (keys + 63) // 64 * 64)         # to whole 64-key blocks
            self.split_L = max(64, int(split_local) // 64 * 64)
        else:
            self.split_L = self.split
        # documents: each its own pool and block table, canonical positions,
        # request offset delta (RedKnot-MLA section 2: segmented reuse; the
        # per-document states merge like the pieces of one document)
        self.docs = [dict(pool=_bf16(d["pool"], device), bt=_i32(d["block_table"], device),
                          num_blocks=int(d["pool"].shape[0]), L=int(d["L"]), delta=int(d["delta"]))
                     for d in prob.documents()]
        self.Ldoc = sum(d["L"] for d in self.docs)
        self.T = prob.T
        self.P = int(len(prot_rows))
        self.d_mid = prob.WaL.shape[1]
        self.d_model = prob.Wb.shape[1]
        self.q = _bf16(prob.q, device)
        self.q_rel = torch.empty_like(self.q)
        self.w_t = pack_weight(prob.W, device)
        # the original kv_b_proj layout (W_UK columns K-contiguous per output
        # row) for the query absorption of the Local heads
        self.W = _bf16(prob.W, device) if self.absorbed else None
        if self.fallback is not None:
            self.art = torch.zeros((max(self.T, 1), max(self.HL, 1), D_V), dtype=torch.bfloat16, device=device)
        elif artifact is not None:
            self.art = artifact.out
        else:
            self.art = _bf16(prob.art_out, device)
        self.prot = _i32(prot_rows, device)
        self.wa_t = pack_weight(np.concatenate([prob.WaL, prob.WaG], axis=0), device)
        self.wb_t = pack_weight(prob.Wb, device)
        T, P = self.T, self.P
        prot = prot_rows
        # chunk plan; piece i of the document is split (chunk c, piece j)
        self.chunks = []
        n_pieces = n_pieces_L = 0
        for di, doc in enumerate(self.docs):
          for s0 in range(0, doc["L"], self.S):
            n = min(self.S, doc["L"] - s0)
            bounds = list(range(0, n, self.split)) + [n]
            k = len(bounds) - 1
            bounds_L = list(range(0, n, self.split_L)) + [n]
            kL = len(bounds_L) - 1
            self.chunks.append(dict(
                doc=di, start=_i32([s0], device), len=_i32([n], device), cu=_i32([0, n], device), n=n,
                pieces=k, first=n_pieces, cu_k=_i32(bounds, device),
                pieces_L=kL, first_L=n_pieces_L, cu_kL=_i32(bounds_L, device),
                cu_qG=_i32(np.arange(k + 1) * T, device), rid_G=_i32(np.tile(np.arange(T), k), device),
                cu_qL=_i32(np.arange(kL + 1) * P, device), rid_L=_i32(np.tile(prot, kL), device)))
            n_pieces += k
            n_pieces_L += kL
        if not self.chunks:
            # no document keys at all: one empty chunk, whose attention writes
            # the empty state (out 0, lse -inf) for every row
            self.chunks.append(dict(
                doc=0, start=_i32([0], device), len=_i32([0], device), cu=_i32([0, 0], device), n=0,
                pieces=1, first=0, cu_k=_i32([0, 0], device), pieces_L=1, first_L=0, cu_kL=_i32([0, 0], device),
                cu_qG=_i32([0, T], device), rid_G=_i32(np.arange(T), device),
                cu_qL=_i32([0, P], device), rid_L=_i32(prot, device)))
            n_pieces = n_pieces_L = 1
        self.max_chunk = max([c["n"] for c in self.chunks] + [1])
        self.n_pieces = n_pieces
        self.n_pieces_L = n_pieces_L
        HL, HG = self.HL, self.HG
        # heads whose k_nope / v are decompressed: all of them, or only the
        # Global ones when the Local rows take the absorbed form
        self.kv_h0 = HL if self.absorbed else 0
        n_kv = H - self.kv_h0
        S = self.max_chunk
        self.lat_ws = torch.empty((S, D_LAT), dtype=torch.bfloat16, device=device)
        self.k_ws = torch.empty((max(n_kv, 1), S, D_V), dtype=torch.bfloat16, device=device)
        self.v_ws = torch.empty((max(n_kv, 1), S, D_V), dtype=torch.bfloat16, device=device)
        self.hstride = S * D_V
        f32, bf = torch.float32, torch.bfloat16
        # partial states of every piece, fp32: [pieces * rows, heads, 128]
        self.part_G = torch.empty((max(n_pieces * T, 1), max(HG, 1), D_V), dtype=f32, device=device)
        self.partl_G = torch.empty((max(n_pieces * T, 1), max(HG, 1)), dtype=f32, device=device)
        if self.absorbed:
            # absorbed Local rows: R = HL * P query rows (head-major), 512-wide
            # latent states viewed as four 128-wide states for the merges
            R = HL * P
            self.q_abs = torch.empty((max(R, 1), D_LAT), dtype=bf, device=device)
            self.part_L = torch.empty((max(n_pieces_L * R, 1), 4, D_V), dtype=f32, device=device)
            self.partl_L = torch.empty((max(n_pieces_L * R, 1), 4), dtype=f32, device=device)
            self.olat_L = torch.empty((max(R, 1), 4, D_V), dtype=bf, device=device)
            self.lse4_L = torch.empty((max(R, 1), 4), dtype=f32, device=device)
        else:
            self.part_L = torch.empty((max(n_pieces_L * P, 1), max(HL, 1), D_V), dtype=f32, device=device)
            self.partl_L = torch.empty((max(n_pieces_L * P, 1), max(HL, 1)), dtype=f32, device=device)
        self.glob_out = torch.empty((T, HG, D_V), dtype=bf, device=device)
        self.lse_G = torch.empty((T, HG), dtype=f32, device=device)
        self.rec_out = torch.empty((max(P, 1), HL, D_V), dtype=bf, device=device)
        if not self.absorbed:
            self._lse_L = torch.empty((max(P, 1), HL), dtype=f32, device=device)
        self.z = torch.empty((T, self.d_mid), dtype=bf, device=device)
        self.y = torch.empty((T, self.d_model), dtype=bf, device=device)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=device)

    @property
    def lse_L(self):
        """lse of the protected rows of the Local heads, [P, HL]."""
        if self.absorbed:
            return self.lse4_L[:, 0].reshape(self.HL, self.P).t()
        return self._lse_L

    def _attn_pieces(self, ch, h0, h1, n_rows, cu_q, rid, part, partl, fin, finl, stream, local=False):
        """Attention of heads [h0, h1) for the query rows rid over every piece
        of chunk ch: piece j's state goes to rows (first + j) * n_rows of the
        fp32 partial buffers, or straight to the bf16 result when the whole
        document is one piece."""
        Hs = h1 - h0
        pieces, first, cu_k, total = ((ch["pieces_L"], ch["first_L"], ch["cu_kL"], self.n_pieces_L) if local
                                      else (ch["pieces"], ch["first"], ch["cu_k"], self.n_pieces))
        if total == 1:
            out, odt, lse = fin, L.DTYPE_BF16, finl
        else:
            row0 = first * n_rows
            out, odt, lse = part[row0:], L.DTYPE_FP32, partl[row0:]
        slab = h0 - self.kv_h0
        L.mla_prefill_attn(self.q_rel, self.H * D_QK, self.H, h0, h1, self.k_ws[slab], self.hstride,
                           self.v_ws[slab], self.hstride, self.lat_ws, D_LAT, cu_q, cu_k, rid,
                           pieces, n_rows, self.prob.scale, 0, out, odt, Hs * D_V, lse, Hs, stream)

    def _absorbed_pieces(self, ch, stream):
        """Absorbed-form attention of the HL * P Local query rows over every
        Local piece of chunk ch (fp32 partial states, or the bf16 result when
        the whole document is one piece)."""
        R = self.HL * self.P
        if self.n_pieces_L == 1:
            out, odt, lse = self.olat_L, L.DTYPE_BF16, self.lse4_L
        else:
            row0 = ch["first_L"] * R
            out, odt, lse = self.part_L[row0:], L.DTYPE_FP32, self.partl_L[row0:]
        L.mla_absorbed_attn(self.q_abs, R, self.lat_ws, D_LAT, ch["cu_kL"], ch["pieces_L"], self.prob.scale,
                            out, odt, lse, stream)

    def _merge_tree(self, part, partl, n_rows, fin, finl, stream, n):
        """merge="tree": merge the n > 1 partial states of every row into
        (fin, finl) by a tree of pairwise merges, where each level merges the
        first half of the remaining pieces with the last half in place (fp32;
        an odd middle piece waits for the next level) and the last level
        writes the bf16 result. (The default merges all pieces, of the
        Global and the Local rows together, in one mla_merge_states_sets
        launch.)"""
        heads = part.shape[1]
        while n > 1:
            h = n // 2
            m = n - h
            a, al = part[:h * n_rows], partl[:h * n_rows]
            b, bl = part[m * n_rows:], partl[m * n_rows:]
            if n == 2:
                out, odt, lo = fin, L.DTYPE_BF16, finl
            else:
                out, odt, lo = a, L.DTYPE_FP32, al
            L.mla_merge_states(a, L.DTYPE_FP32, al, b, L.DTYPE_FP32, bl, h * n_rows * heads, out, odt,
                               lo, stream)
            n = m

    def run(self, stream=None, timer=None, check=True):
        """One reuse step; returns y. check as in ChunkedPrefill.run."""
        y = self._run(stream, timer)
        self._finish(check, stream)
        return y

    def _run(self, stream, timer):
        p = self.prob
        H, HL, HG, T, P = self.H, self.HL, self.HG, self.T, self.P
        cur_doc = -1
        for ch in self.chunks:
            doc = self.docs[ch["doc"]]
            if ch["doc"] != cur_doc:
                # queries into this document's canonical frame (and, for the
                # absorbed Local rows, their absorbed form from the relocated
                # rope part)
                cur_doc = ch["doc"]
                with _span(timer, "relocate"):
                    L.mla_rope_relocate_q(self.q, self.q_rel, H * D_QK, T, H, doc["delta"], p.rope_base,
                                          L.ROPE_INTERLEAVED, stream)
                if self.absorbed and HL > 0 and P > 0:
                    with _span(timer, "absorb"):
                        L.mla_absorb_q(self.q_rel, H * D_QK, H, 0, HL, self.prot, P, self.W, H, self.q_abs,
                                       stream)
            with _span(timer, "gather"):
                L.mla_gather_context(doc["pool"], L.DTYPE_BF16, doc["num_blocks"], doc["bt"], doc["bt"].shape[1],
                                     ch["start"], ch["len"], ch["cu"], 1, ch["n"], self.lat_ws,
                                     self.dev_status, stream)
            if self.kv_h0 < H:
                with _span(timer, "decompress"):
                    L.mla_decompress(self.lat_ws, D_LAT, None, ch["n"], self.w_t, H, self.kv_h0, H, self.k_ws,
                                     self.hstride, self.v_ws, self.hstride, stream)
            if HG > 0 and T > 0:
                with _span(timer, "attn_global"):
                    self._attn_pieces(ch, HL, H, T, ch["cu_qG"], ch["rid_G"], self.part_G, self.partl_G,
                                      self.glob_out, self.lse_G, stream)
            if HL > 0 and P > 0:
                with _span(timer, "attn_local"):
                    if self.absorbed:
                        self._absorbed_pieces(ch, stream)
                    else:
                        self._attn_pieces(ch, 0, HL, P, ch["cu_qL"], ch["rid_L"], self.part_L,
                                          self.partl_L, self.rec_out, self._lse_L, stream, local=True)
        with _span(timer, "merge"):
            merges = []          # (part, partl, rows of the partial buffers, result, its lse, pieces)
            if HG > 0 and T > 0:
                merges.append((self.part_G, self.partl_G, T, self.glob_out, self.lse_G, self.n_pieces))
            if HL > 0 and P > 0:
                if self.absorbed:
                    merges.append((self.part_L, self.partl_L, HL * P, self.olat_L, self.lse4_L, self.n_pieces_L))
                else:
                    merges.append((self.part_L, self.partl_L, P, self.rec_out, self._lse_L, self.n_pieces_L))
            merges = [m for m in merges if m[5] > 1]   # one piece was written to its result directly
            if self.merge_mode == "one_pass":
                # the Global and the Local merges in one launch
                if merges:
                    L.mla_merge_states_sets([(part, partl, n, rows * part.shape[1], fin, finl)
                                             for part, partl, rows, fin, finl, n in merges],
                                            L.DTYPE_FP32, L.DTYPE_BF16, stream)
            else:
                for part, partl, rows, fin, finl, n in merges:
                    self._merge_tree(part, partl, rows, fin, finl, stream, n)
        if self.absorbed and HL > 0 and P > 0:
            with _span(timer, "absorb"):
                L.mla_absorb_out(self.olat_L, P, self.w_t, H, 0, HL, self.rec_out, HL * D_V, stream)
        with _span(timer, "projection"):
            L.mla_head_partition_merge(self.art, self.rec_out, self.prot, P, self.glob_out, self.wa_t,
                                       self.wb_t, T, HL, HG, self.d_mid, self.d_model, self.z, self.y,
                                       stream)
        return self.y

    def work(self) -> dict:
        """Algorithmic work of one run, in the same units as ChunkedPrefill.work.
        Merges: the one-pass merge reads every piece's fp32 state once
        (516 B per piece and (row, head)) and writes one bf16 state (260 B);
        the pairwise tree makes n_pieces - 1 merges per (row, head), each
        reading two fp32 states (2 * 516 B) and writing one (516 B), the last
        one in bf16 (260 B)."""
        H, HL, HG, T, P, Ld = self.H, self.HL, self.HG, self.T, self.P, self.Ldoc
        n = self.n_pieces
        if self.absorbed:
            # Global rows: decompressed form; Local protected rows: absorbed
            # form, 2 * 576 + 2 * 512 flop per (row, key, head), plus the
            # query absorption and the W_UV product (2 * 128 * 512 each per
            # (row, head)); merges of 512-wide states (4 x 128)
            merge_rows = T * HG + 4 * P * HL
            dec_heads = HG
            local = 2176 * Ld * P * HL
            absorb = 2 * (2 * 128 * 512) * P * HL
        else:
            merge_rows = T * HG + P * HL
            dec_heads = H
            local = 640 * Ld * P * HL
            absorb = 0
        def tree(rows, k):
            if k <= 1:
                return 0
            if self.merge_mode == "one_pass":
                return rows * (k * 516 + 260)
            return rows * ((k - 2) * 3 * 516 + (2 * 516 + 260))
        merge_bytes = tree(T * HG, n) + tree(merge_rows - T * HG, self.n_pieces_L)
        glob = 640 * Ld * T * HG
        return dict(
            dec_flops=2 * 512 * 256 * dec_heads * Ld,
            attn_flops=glob + local,
            global_attn_flops=glob,
            local_attn_flops=local,
            absorb_flops=absorb,
            proj_flops=2 * T * ((HL + HG) * 128 * self.d_mid + self.d_mid * self.d_model),
            relocate_bytes=T * H * 768 * len(self.docs),   # per document, out of place: q head row read + written
            merge_bytes=int(merge_bytes),
            gather_tokens=Ld, gather_bytes=Ld * 2304, new_tokens=T, ctx_tokens=Ld,
        )


class Artifact:
    """An offline Local-head artifact: out [R, HL, 128] bf16 and lse [R, HL]
    fp32 on the device, with its description (ArtifactMeta)."""

    def __init__(self, out, lse, meta):
        self.out, self.lse, self.meta = out, lse, meta


def artifact_meta(tokens, generation, H, n_local, rope_base=10000.0, n_layers=1, layers=(0,)):
    """Description of a document's artifact, or of what a request needs from
    it: the token binding (mla_token_hash), the profile and the layers."""
    mask = 0
    for l in layers:
        mask |= 1 << int(l)
    return L.ArtifactMeta(generation=int(generation), token_hash=L.mla_token_hash(tokens),
                          n_tokens=int(len(tokens)), n_heads=int(H), n_local=int(n_local), d_c=512,
                          d_rope=64, d_nope=128, d_v=D_V, rope_base=float(rope_base), n_layers=int(n_layers),
                          reserved=0, layer_mask=mask)


class ArtifactBuilder(_DeviceStatus):
    """MLA-Off: one document processed alone at canonical position zero,
    Local heads only (RedKnot-MLA Abstract and section 2).

    Rows: q [R, H, 192] bf16 with rope parts at canonical positions. With
    doc_rows, rows 0..L-1 are the document's own tokens (row t sees keys
    0..t) and later rows follow the document (they see all of it); without,
    every row follows the document.

    Per key chunk [s0, s0 + n): gather, decompression of the Local heads,
    then two attention passes over the chunk's keys. Rows past the chunk
    (document rows from s0 + n on, then the following rows) attend to all of
    it, merged into an fp32 running state (the last chunk writes their bf16
    result). The chunk's own document rows attend causally (n_q = n_k = n,
    bottom-right aligned, so row s0 + i sees keys s0..s0 + i), merged with
    their running state and written as the final bf16 result: no later chunk
    reaches them. One chunk holding the whole document needs no merges.
    """

    def __init__(self, pool, block_table, L_doc, q, W_bits, H, n_local, scale, doc_rows=True, chunk=None,
                 device="cuda", tokens=None, generation=0, rope_base=10000.0, n_layers=1, layer=0):
        self.device = device
        self.H, self.HL = int(H), int(n_local)
        self.L = int(L_doc)
        self.doc_rows = bool(doc_rows)
        self.scale = float(scale)
        self.pool = pool if isinstance(pool, torch.Tensor) else _bf16(pool, device)
        self.bt = block_table if isinstance(block_table, torch.Tensor) else _i32(block_table, device)
        self.q = q if isinstance(q, torch.Tensor) else _bf16(q, device)
        self.R = int(self.q.shape[0])
        if self.doc_rows and self.R < self.L:
            raise ValueError("ArtifactBuilder: with doc_rows the first L rows are the document's tokens")
        self.w_t = pack_weight(W_bits, device)
        self.S = max(1, min(int(chunk or self.L), max(self.L, 1)))
        self.chunks = []
        for s0 in range(0, self.L, self.S):
            n = min(self.S, self.L - s0)
            a0 = s0 + n if self.doc_rows else 0          # first row past the chunk
            self.chunks.append(dict(s0=s0, n=n, a0=a0, start=_i32([s0], device), len=_i32([n], device),
                                    cu=_i32([0, n], device), cu_after=_i32([0, self.R - a0], device)))
        S, HL = self.S, self.HL
        bf, f32 = torch.bfloat16, torch.float32
        self.lat_ws = torch.empty((S, D_LAT), dtype=bf, device=device)
        self.k_ws = torch.empty((max(HL, 1), S, D_V), dtype=bf, device=device)
        self.v_ws = torch.empty((max(HL, 1), S, D_V), dtype=bf, device=device)
        self.hstride = S * D_V
        self.out = torch.empty((max(self.R, 1), max(HL, 1), D_V), dtype=bf, device=device)
        self.lse = torch.empty((max(self.R, 1), max(HL, 1)), dtype=f32, device=device)
        if len(self.chunks) > 1:
            self.acc = torch.empty((self.R, HL, D_V), dtype=f32, device=device)
            self.acc_lse = torch.empty((self.R, HL), dtype=f32, device=device)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=device)
        self._cu_rows = _i32([0, self.R], device)
        self._cu_none = _i32([0, 0], device)
        self.meta = artifact_meta(tokens if tokens is not None else np.zeros(0, np.int32), generation, H,
                                  n_local, rope_base, n_layers, (layer,))
        if tokens is not None and len(tokens) != self.L:
            raise ValueError("ArtifactBuilder: tokens must hold the document's L ids")

    @classmethod
    def from_problem(cls, ap, device="cuda", chunk=None):
        return cls(ap.pool, ap.block_table, ap.L, ap.q, ap.W, ap.H, ap.n_local, ap.scale, ap.doc_rows,
                   chunk or ap.chunk, device, ap.tokens, ap.generation, ap.rope_base)

    def _attn(self, r0, n_rows, cu_q, cu_k, causal, merge, final, stream):
        H, HL = self.H, self.HL
        q = self.q[r0:]
        out, odt, lse = ((self.out[r0:], L.DTYPE_BF16, self.lse[r0:]) if final
                         else (self.acc[r0:], L.DTYPE_FP32, self.acc_lse[r0:]))
        common = (q, H * D_QK, H, 0, HL, self.k_ws, self.hstride, self.v_ws, self.hstride, self.lat_ws, D_LAT,
                  cu_q, cu_k, None, 1, n_rows, self.scale, int(causal))
        if merge:
            L.mla_prefill_attn_merge(*common, self.acc[r0:], HL * D_V, self.acc_lse[r0:], HL, out, odt, HL * D_V,
                                     lse, HL, stream)
        else:
            L.mla_prefill_attn(*common, out, odt, HL * D_V, lse, HL, stream)

    def run(self, stream=None, timer=None, check=True) -> Artifact:
        """Build the artifact. check: wait for the build and raise before the
        Artifact is returned if the gather met a block id outside the pool
        (an artifact built from zero records must not be handed out);
        skipped under graph capture."""
        art = self._run(stream, timer)
        self._finish(check, stream)
        return art

    def _run(self, stream, timer) -> Artifact:
        n_ch = len(self.chunks)
        if n_ch == 0 and self.R > 0 and self.HL > 0:
            # an empty document: every row sees no key, so the attention over
            # an empty key range writes out = 0 and lse = -inf
            with _span(timer, "attn_full"):
                L.mla_prefill_attn(self.q, self.H * D_QK, self.H, 0, self.HL, self.k_ws, self.hstride, self.v_ws,
                                   self.hstride, self.lat_ws, D_LAT, self._cu_rows, self._cu_none, None, 1, self.R,
                                   self.scale, 0, self.out, L.DTYPE_BF16, self.HL * D_V, self.lse, self.HL, stream)
        for ci, ch in enumerate(self.chunks):
            first, last = ci == 0, ci == n_ch - 1
            with _span(timer, "gather"):
                L.mla_gather_context(self.pool, L.DTYPE_BF16, int(self.pool.shape[0]), self.bt, self.bt.shape[1],
                                     ch["start"], ch["len"], ch["cu"], 1, ch["n"], self.lat_ws, self.dev_status,
                                     stream)
            if self.HL == 0:
                continue
            with _span(timer, "decompress"):
                L.mla_decompress(self.lat_ws, D_LAT, None, ch["n"], self.w_t, self.H, 0, self.HL, self.k_ws,
                                 self.hstride, self.v_ws, self.hstride, stream)
            n_after = self.R - ch["a0"]
            if n_after > 0:
                with _span(timer, "attn_full"):
                    self._attn(ch["a0"], n_after, ch["cu_after"], ch["cu"], False, merge=not first,
                               final=last, stream=stream)
            if self.doc_rows:
                with _span(timer, "attn_causal"):
                    self._attn(ch["s0"], ch["n"], ch["cu"], ch["cu"], True, merge=not first, final=True,
                               stream=stream)
        return Artifact(self.out[:self.R, :self.HL], self.lse[:self.R, :self.HL], self.meta)

    def work(self) -> dict:
        """Algorithmic work of one build: decompression of the Local heads
        over the document (2 * 512 * 256 flop per (token, head)) and 640 flop
        per visible (row, key, head)."""
        L_, HL = self.L, self.HL
        n_doc = L_ if self.doc_rows else 0
        pairs = n_doc * (n_doc + 1) // 2 + (self.R - n_doc) * L_
        causal = sum(c["n"] * (c["n"] + 1) // 2 for c in self.chunks) if self.doc_rows else 0
        return dict(dec_flops=2 * 512 * 256 * HL * L_, attn_flops=640 * HL * pairs,
                    causal_attn_flops=640 * HL * causal, full_attn_flops=640 * HL * (pairs - causal),
                    gather_bytes=L_ * 2304, rows=self.R, doc_tokens=L_)


class GraphStep:
    """One step of a driver (ChunkedPrefill, ReusePrefill, ArtifactBuilder)
    captured once into a HIP graph and replayed: the same kernels on the same
    buffers, without a host launch per kernel. The driver's buffers must stay
    alive and in place while the graph is used. Capture runs on a side stream
    (as torch requires); replay() enqueues on the current stream."""

    def __init__(self, driver, warmup=1):
        self.driver = driver
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                driver.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            driver.run()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()

    run = replay
