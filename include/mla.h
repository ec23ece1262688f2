/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA chunked-prefill library.
 *
 * The library computes multi-head latent attention (MLA) prefill over a
 * paged cache that stores, per token and layer, one packed record of the
 * 512-wide compressed latent c_kv followed by the 64-wide rope key k_rope
 * (576 elements), in 64-token blocks. The packed record is never split per
 * head: per-head keys and values are decompressed from it through kv_b_proj
 * chunk by chunk, and chunk results are merged by log-sum-exp.
 *
 * Pages the operations follow:
 *   [DSMLA]   "DeepSeek MLA -- Prefix Cache and Chunked Prefill" notes,
 *             section 4.2 (context + extend stages), 4.3 (merge_attn_states),
 *             4.4 (_compute_prefill_context chunk loop), 5.2 (576-element
 *             packed record).
 *   [PAGED]   "PagedAttention assumed MHA. DeepSeek-V4 says that assumption
 *             is broken.", sections "Block size is not a tuning knob here"
 *             (64-token blocks) and "What DeepSeek-V4 breaks" (bf16 rope next
 *             to fp8 content within one block).
 *   [REDKNOT] "RedKnot-MLA: Multi-Head Offline-Online Reuse for DeepSeek-V4
 *             Long-Context Serving", Abstract and sections 1-3 (query-side
 *             RoPE relocation, Local/Global heads, protected rows, sliced
 *             projection before one shared output projection, Equation 4).
 *
 * Conventions for every entry point:
 *   - Pointers named dev_* or typed as tensors are DEVICE pointers to memory
 *     the caller owns (allocated by the caller, e.g. through PyTorch). The
 *     library never allocates, frees or synchronises; every call only
 *     enqueues kernels.
 *   - stream is a hipStream_t (passed as void*; NULL = the null stream).
 *     Every call only enqueues kernels on that stream and returns; results
 *     are ready when the stream reaches that point.
 *   - Return value: MLA_OK, or a negative mla_status. Arguments are checked
 *     on the host before anything is enqueued; on error nothing is enqueued
 *     and mla_last_error() describes the problem (thread-local string).
 *     A problem whose grid would exceed the launch limits (2^31 - 1
 *     workgroups, or 65535 in a second grid dimension) is refused, never
 *     truncated: with MLA_ERR_INVALID_ARG ("too large") by the argument
 *     checks, or with MLA_ERR_LAUNCH where the runtime's own check of the
 *     grid rejects it; split such a problem over several calls.
 *   - Geometry is fixed: d_c = 512, d_rope = 64, d_nope = d_v = 128,
 *     d_qk = 192, block = 64 tokens. Strides are in ELEMENTS of the stated
 *     dtype. Base pointers must be 16-byte aligned and row strides multiples
 *     of 8 elements (16 bytes for bf16).
 *   - bf16 is bfloat16 (top half of IEEE fp32); fp8 is OCP E4M3FN (max 448);
 *     fp32 is IEEE single.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad stride/alignment */
  MLA_ERR_UNSUPPORTED = -2,   /* valid but not implemented (dtype, geometry)  */
  MLA_ERR_LAUNCH = -3,        /* the HIP runtime refused the launch           */
  MLA_ERR_OUT_OF_RANGE = -4   /* device-side: a block id outside the pool     */
} mla_status;

typedef enum {
  MLA_DTYPE_BF16 = 0,
  MLA_DTYPE_FP8_E4M3 = 1,
  MLA_DTYPE_FP32 = 2
} mla_dtype;

typedef enum {
  MLA_ROPE_INTERLEAVED = 0,   /* pair k = elements (2k, 2k+1)  */
  MLA_ROPE_HALF = 1           /* pair k = elements (k, k + 32) */
} mla_rope_pairing;

/* Message describing the last error returned on this thread ("" if none). */
const char* mla_last_error(void);

/* ABI version, currently 2. */
int mla_abi_version(void);

/*
 * mla_gather_context -- [DSMLA] 4.4 step 1 (_gather_cache); block addressing
 * per [PAGED] "Block size is not a tuning knob here".
 *
 * For each request b in [0, batch), copies the latent records of its tokens
 * t in [chunk_start[b], chunk_start[b] + chunk_len[b]) into consecutive rows
 * [cu_out[b], cu_out[b] + chunk_len[b]) of out_latent. Token t lives in
 * physical block block_table[b * bt_stride + t / 64] at slot t % 64.
 *
 *   pool        device; cache_dtype == MLA_DTYPE_BF16: bf16 [num_blocks][64][576]
 *               (record = c_kv[512] then k_rope[64]).
 *               cache_dtype == MLA_DTYPE_FP8_E4M3: bytes [num_blocks][41216]; per
 *               block c_kv codes [64][512] at byte 0, k_rope bf16 [64][64] at
 *               byte 32768, per-token fp32 scale [64] at byte 40960.
 *   block_table device int32 [batch][bt_stride].
 *   chunk_start, chunk_len, cu_out  device int32 [batch], [batch], [batch+1].
 *   batch       host, <= 65535.
 *   max_len     host; >= every chunk_len[b] (sizes the launch).
 *   out_latent  device bf16 [cu_out[batch]][576], row stride 576.
 *   dev_status  device int32 or NULL. A block id outside [0, num_blocks)
 *               makes the kernel write zeros for that token and store
 *               MLA_ERR_OUT_OF_RANGE into *dev_status (never cleared by the
 *               library; the caller zeroes it).
 * bf16 cache: out is a bit copy. fp8 cache: c_kv out = bf16_rne(fp32
 * product of the decoded code and the token's scale), k_rope copied.
 */
int mla_gather_context(const void* pool, int cache_dtype, int num_blocks,
                       const int32_t* block_table, int64_t bt_stride,
                       const int32_t* chunk_start, const int32_t* chunk_len,
                       const int32_t* cu_out, int batch, int max_len,
                       void* out_latent, int32_t* dev_status, void* stream);

/*
 * mla_gather_context_fp8_raw -- mla_gather_context for an fp8 cache without
 * dequantisation ([DSMLA] 4.4 step 1 with the fp8 storage of 2.2): the
 * decompression then reads the codes itself (mla_decompress with row_scale),
 * so c_kv moves as 512 bytes per token instead of 1024.
 *
 * Arguments as mla_gather_context (pool is the fp8 layout), and for output
 * row o = cu_out[b] + (t - chunk_start[b]) of token t:
 *   out_latent  device, rows of 576 bf16 elements (1152 bytes): bytes
 *               0..511 of row o are the token's 512 E4M3FN codes of c_kv,
 *               copied; elements 512..575 its bf16 k_rope, copied; bytes
 *               512..1023 are not written.
 *   out_scale   device fp32 [cu_out[batch]]: out_scale[o] is the token's scale.
 * A block id outside [0, num_blocks) writes zero codes, scale 0 and zero
 * k_rope for that token and stores MLA_ERR_OUT_OF_RANGE into *dev_status.
 * Pointers 16-byte aligned.
 */
int mla_gather_context_fp8_raw(const void* pool, int num_blocks, const int32_t* block_table,
                               int64_t bt_stride, const int32_t* chunk_start, const int32_t* chunk_len,
                               const int32_t* cu_out, int batch, int max_len, void* out_latent,
                               float* out_scale, int32_t* dev_status, void* stream);

/*
 * mla_pack_weight_t -- weight layout transform done once at load time (not
 * part of the per-prefill path): out[n][k] = w[k][n] for a bf16 matrix
 * w [K][N] (row-major). Used to store kv_b_proj [512][H*256] and the sliced
 * and shared output projections as [N][K], so that both MFMA operands read
 * contiguous K. K and N must be multiples of 8.
 */
int mla_pack_weight_t(const void* w, int K, int N, void* out, void* stream);

/*
 * mla_cache_append -- the cache write path ([PAGED] "Position independence
 * beats prefix matching": new records are written into 64-token blocks that
 * are sealed once full; [DSMLA] 2.2: fp8 storage of the latent).
 *
 * Token i < n_b = cu_new[b+1] - cu_new[b] of request b (record row
 * cu_new[b] + i of latent_new, [c_kv 512 | k_rope 64] bf16, row stride
 * ld_latent elements) is written at position t = pos0[b] + i: block
 * block_table[b * bt_stride + t / 64], slot t % 64.
 *   cache_dtype = MLA_DTYPE_BF16: pool [num_blocks][64][576] bf16, the
 *     record is copied.
 *   cache_dtype = MLA_DTYPE_FP8_E4M3: pool blocks of 41216 bytes, codes
 *     [64][512] | k_rope [64][64] bf16 | scale [64] fp32. scale =
 *     fp32(max|c_kv|) / 448 and code = E4M3FN(clamp(c_kv / scale, +-448)),
 *     each division correctly rounded and the encoding round-to-nearest-
 *     even (reading R14); a record of zeros gets scale 0 and +0 codes. k_rope
 *     is copied as bf16.
 * A position with t < 0 or t / 64 >= bt_stride, or a block id outside
 * [0, num_blocks), is skipped and sets *dev_status = MLA_ERR_OUT_OF_RANGE
 * (dev_status may be NULL). No other byte of the pool is written. All
 * pointers are device memory; pool, block_table, pos0 and cu_new are int32
 * or byte arrays owned by the caller; max_new (host) >= every n_b sizes the
 * launch. Positions of one call must be distinct.
 */
int mla_cache_append(void* pool, int cache_dtype, int num_blocks, const int32_t* block_table,
                     int64_t bt_stride, const int32_t* pos0, const int32_t* cu_new, int batch,
                     int max_new, const void* latent_new, int64_t ld_latent, int32_t* dev_status,
                     void* stream);

/*
 * mla_decompress -- [DSMLA] 4.4 step 2: kv = c_kv . kv_b_proj, split into
 * per-head k_nope and v.
 *
 *   latent      device, rows of ld_latent bf16 elements (2 * ld_latent
 *               bytes), n_tokens rows. Without row_scale: c_kv = elements
 *               0..511 (bf16). With row_scale: c_kv of row t is
 *               row_scale[t] times the E4M3FN codes in bytes 0..511 of the
 *               row (as written by mla_gather_context_fp8_raw, [DSMLA] 2.2);
 *               the codes enter the bf16 products exactly and the scale
 *               multiplies the fp32 sums, before the one rounding to bf16.
 *   row_scale   device fp32 [n_tokens] or NULL (4-byte aligned).
 *   w_t         device bf16 [H_total*256][512]: kv_b_proj packed by
 *               mla_pack_weight_t (row j = output column j; columns
 *               [0, H*128) are W_UK of heads 0..H-1, [H*128, H*256) W_UV).
 *   heads       [h_begin, h_end) of H_total are produced, hs = h - h_begin.
 *   k_nope      device bf16; k_nope[hs * k_head_stride + t * 128 + d].
 *   v           device bf16; v[hs * v_head_stride + t * 128 + d].
 *               Head strides >= n_tokens * 128 (head-major, so one head's
 *               keys of a chunk are contiguous).
 * fp32 accumulation, one bf16 rounding of each output.
 */
int mla_decompress(const void* latent, int64_t ld_latent, const float* row_scale, int n_tokens,
                   const void* w_t, int H_total, int h_begin, int h_end,
                   void* k_nope, int64_t k_head_stride,
                   void* v, int64_t v_head_stride, void* stream);

/*
 * mla_prefill_attn -- [DSMLA] 4.4 steps 3-4 (attention returning (out, lse))
 * for the context pass (causal = 0) and the extend pass (causal = 1) of
 * [DSMLA] 4.2.
 *
 * For request b: logical query rows i in [0, n_q), n_q = cu_q[b+1]-cu_q[b];
 * keys t in [cu_k[b], cu_k[b+1]), n_k = cu_k[b+1]-cu_k[b]. For head h in
 * [h_begin, h_end) (hs = h - h_begin):
 *   s_t = scale * (q_nope . k_nope[hs][t] + q_rope . k_rope[t])
 * where q = q[p * q_row_stride + h * 192 + (0..191)] (nope first) with
 * p = q_row_ids ? q_row_ids[cu_q[b] + i] : cu_q[b] + i, and k_rope[t] =
 * latent[t * ld_latent + 512 + (0..63)] shared by every head. causal = 1
 * keeps key t iff (t - cu_k[b]) <= i + n_k - n_q (bottom-right aligned).
 *   out[(cu_q[b]+i) * out_row_stride + hs * 128 + d] = sum_t softmax(s)_t v[t][d]
 *   lse[(cu_q[b]+i) * lse_row_stride + hs]            = ln sum_t e^{s_t}
 * with v[t] = v[hs * v_head_stride + t * 128 + (0..127)].
 * A row with no visible key gets out = 0 and lse = -inf.
 *   q          device bf16; k_nope / v as written by mla_decompress
 *              (row t of head hs at hs * head_stride + t * 128).
 *   latent     device bf16 rows of ld_latent elements, ld_latent a multiple
 *              of 8 in [576, 2^17].
 *   out_dtype  MLA_DTYPE_BF16 or MLA_DTYPE_FP32.
 *   max_q      host; >= every n_q (sizes the launch).
 */
int mla_prefill_attn(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                     const void* k_nope, int64_t k_head_stride,
                     const void* v, int64_t v_head_stride,
                     const void* latent, int64_t ld_latent,
                     const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_row_ids,
                     int batch, int max_q, float scale, int causal,
                     void* out, int out_dtype, int64_t out_row_stride,
                     float* lse, int64_t lse_row_stride, void* stream);

/*
 * mla_prefill_attn_merge -- mla_prefill_attn followed by the log-sum-exp
 * merge of [DSMLA] 4.3 with a previous state, in one pass: the chunk loop of
 * [DSMLA] 4.4 merges every chunk's (out, lse) into the running state, and
 * here that merge happens in the attention epilogue, in fp32, before the
 * result is rounded.
 *
 * Arguments as mla_prefill_attn, plus the previous state of the same rows
 * and heads (fp32, 16-byte aligned):
 *   prev_out[(cu_q[b]+i) * prev_row_stride + hs * 128 + d]
 *   prev_lse[(cu_q[b]+i) * prev_lse_row_stride + hs]
 * The result (out, lse) is merge(prev, this pass) as in mla_merge_states: a
 * side with lse = -inf contributes nothing (its out is not read), both -inf
 * give out = 0 and lse = -inf. out and lse may be the previous state itself
 * (same pointers and strides, out_dtype = MLA_DTYPE_FP32): each element is
 * read before it is written, and rows of a request with no keys in this pass
 * are left untouched (the merge with an empty set is the identity). Any
 * other overlap is undefined.
 */
int mla_prefill_attn_merge(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                           const void* k_nope, int64_t k_head_stride,
                           const void* v, int64_t v_head_stride,
                           const void* latent, int64_t ld_latent,
                           const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_row_ids,
                           int batch, int max_q, float scale, int causal,
                           const float* prev_out, int64_t prev_row_stride,
                           const float* prev_lse, int64_t prev_lse_row_stride,
                           void* out, int out_dtype, int64_t out_row_stride,
                           float* lse, int64_t lse_row_stride, void* stream);

/*
 * mla_prefill_attn_2seg -- the last pass of the [DSMLA] 4.4 chunk loop and
 * the causal pass over the new tokens ([DSMLA] 4.2) in one launch: each row
 * attends to the keys of two segments with one online softmax, then (when a
 * previous state is given) is merged into it as in mla_prefill_attn_merge.
 * The result is the plain softmax over the union of both key sets, the
 * same value the two passes and their merge compute, up to rounding order.
 *
 *   segment 1: keys t in [cu_k[b], cu_k[b+1]) of (k_nope, v, latent), all
 *              visible (the chunk's context tokens);
 *   segment 2: keys t in [cu_k2[b], cu_k2[b+1]) of (k_nope2, v2, latent2),
 *              causal: row i sees key t iff (t - cu_k2[b]) <= i + n_k2 - n_q
 *              (the request's own new tokens).
 * Scores, k_rope (columns 512..575 of each segment's latent rows), out and
 * lse as mla_prefill_attn. Either segment may be empty for a request; with
 * prev_out = prev_lse = NULL no merge happens, otherwise both must be given
 * (fp32, as in mla_prefill_attn_merge, with the same aliasing rule).
 * Constraints: ld_latent2 == ld_latent (MLA_ERR_UNSUPPORTED otherwise); no
 * row ids; pointers 16-byte aligned and head strides multiples of 8 as in
 * mla_prefill_attn.
 */
int mla_prefill_attn_2seg(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                          const void* k_nope, int64_t k_head_stride,
                          const void* v, int64_t v_head_stride,
                          const void* latent, int64_t ld_latent, const int32_t* cu_k,
                          const void* k_nope2, int64_t k_head_stride2,
                          const void* v2, int64_t v_head_stride2,
                          const void* latent2, int64_t ld_latent2, const int32_t* cu_k2,
                          const int32_t* cu_q, int batch, int max_q, float scale,
                          const float* prev_out, int64_t prev_row_stride,
                          const float* prev_lse, int64_t prev_lse_row_stride,
                          void* out, int out_dtype, int64_t out_row_stride,
                          float* lse, int64_t lse_row_stride, void* stream);

/*
 * mla_prefill_attn_chunk -- one pass of the [DSMLA] 4.4 chunk loop over a
 * ragged batch in which each request's causal pass over its new tokens
 * ([DSMLA] 4.2) joins the pass of that request's own last context chunk,
 * instead of a separate pass after the loop. For request b:
 *   last[b] == 0: segment 1 only (the chunk's context keys [cu_k[b],
 *                 cu_k[b+1]), all visible); the result is merged into the
 *                 running state (when merge != 0) and written back to
 *                 state / state_lse in fp32;
 *   last[b] != 0: segment 1 and segment 2 (the new tokens' keys [cu_k2[b],
 *                 cu_k2[b+1]), causal as in mla_prefill_attn_2seg) in one
 *                 online softmax, merged into the running state (when
 *                 merge != 0); the final result goes to out (bf16) and its
 *                 lse to state_lse.
 * merge == 0 is the loop's first pass: no state is read. The state is read
 * and written in place (state [rows][...] fp32 with state_row_stride,
 * state_lse fp32 with state_lse_row_stride), so after the request's last
 * pass state_lse holds its final lse. In a merging pass, a request with
 * last[b] == 0 and no key in segment 1 leaves its state untouched (merging
 * an empty key set is the identity), which skips requests whose last pass
 * came earlier; in a first pass (merge == 0) such a request gets the empty
 * state (0, -inf). Final rows leave state untouched, and the other rows out.
 * Everything else (q, segments, strides, scale, cu_q, max_q) as in
 * mla_prefill_attn_2seg; last, state and state_lse must not be NULL.
 */
int mla_prefill_attn_chunk(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                           const void* k_nope, int64_t k_head_stride,
                           const void* v, int64_t v_head_stride,
                           const void* latent, int64_t ld_latent, const int32_t* cu_k,
                           const void* k_nope2, int64_t k_head_stride2,
                           const void* v2, int64_t v_head_stride2,
                           const void* latent2, int64_t ld_latent2, const int32_t* cu_k2,
                           const int32_t* last, const int32_t* cu_q, int batch, int max_q, float scale,
                           int merge, float* state, int64_t state_row_stride,
                           float* state_lse, int64_t state_lse_row_stride,
                           void* out, int64_t out_row_stride, void* stream);

/*
 * Absorbed-form attention ([DSMLA] section 3: W_UK folded into the query,
 * W_UV applied after the attention, every head attends to the shared
 * 576-wide latent), for query sets small next to the key count: the
 * protected rows of the Local heads in [REDKNOT] section 2. Three calls:
 *
 * mla_absorb_q -- for head h in [h_begin, h_end) (hs = h - h_begin) and row
 * i < n_rows (query row p = row_ids[i]):
 *   q_abs[(hs * n_rows + i) * 576 + j] = sum_d q[p][h][d] * kv_b_proj[j][h * 128 + d]
 *                                        for j < 512 (d < 128, nope part)
 *   q_abs[(hs * n_rows + i) * 576 + 512 + r] = q[p][h][128 + r]   (rope part, copied)
 * with q[p][h][e] = q[p * q_row_stride + h * 192 + e], kv_b_proj the bf16
 * [512][H_total * 256] weight in its original layout (W_UK columns first).
 * Accumulation in fp32, q_abs rounded to bf16.
 */
int mla_absorb_q(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                 const int32_t* row_ids, int n_rows, const void* kv_b_proj, int H_total,
                 void* q_abs, void* stream);

/*
 * mla_absorbed_attn -- multi-query attention of R absorbed query rows
 * (q_abs [R][576] bf16) over latent keys, separately for each of `pieces` key
 * ranges [cu_k[b], cu_k[b+1]) of latent (rows of ld_latent elements):
 *   s_t = scale * (q_abs[i] . latent[t][0..575])
 *   o_lat[(b * R + i) * 512 + d] = sum_t softmax(s)_t latent[t][d]     (d < 512)
 *   lse4[(b * R + i) * 4 + k]   = ln sum_t e^{s_t}                     (k < 4)
 * The lse is written four times so that each 512-wide state is also four
 * 128-wide states with their own lse, as mla_merge_states reads them: the
 * pieces of a row merge with mla_merge_states over 4 * R rows. An empty piece
 * gives o_lat = 0 and lse = -inf. out_dtype MLA_DTYPE_BF16 or
 * MLA_DTYPE_FP32.
 */
int mla_absorbed_attn(const void* q_abs, int R, const void* latent, int64_t ld_latent,
                      const int32_t* cu_k, int pieces, float scale, void* out_lat, int out_dtype,
                      float* lse4, void* stream);

/*
 * mla_absorb_out -- out[i * out_row_stride + hs * 128 + e] =
 *   sum_d o_lat[(hs * n_rows + i) * 512 + d] * kv_b_proj[d][H_total * 128 + h * 128 + e]
 * for head h = h_begin + hs, with o_lat bf16 and the weight given packed as
 * by mla_pack_weight_t (w_t [H_total * 256][512]). fp32 accumulation, bf16
 * out.
 */
int mla_absorb_out(const void* o_lat, int n_rows, const void* w_t, int H_total, int h_begin, int h_end,
                   void* out, int64_t out_row_stride, void* stream);

/*
 * mla_merge_states -- [DSMLA] 4.3 (merge_attn_states), with the merged lse
 * m + ln(e^{la-m} + e^{lb-m}) that the chunk loop of 4.4 consumes.
 *
 * rows independent states of 128 values: out_x[r * 128 + d], lse_x[r].
 *   out = (wa * out_a + wb * out_b) / (wa + wb), wa = e^{lse_a - m},
 *   wb = e^{lse_b - m}, m = max(lse_a, lse_b); lse = m + ln(wa + wb).
 * A side with lse = -inf contributes nothing (its out is not read); both
 * -inf gives out = 0, lse = -inf. out may alias out_a or out_b and lse_out
 * may alias lse_a or lse_b (each element is read before it is written).
 * dtype_a, dtype_b, dtype_out: MLA_DTYPE_BF16 or MLA_DTYPE_FP32.
 */
int mla_merge_states(const void* out_a, int dtype_a, const float* lse_a,
                     const void* out_b, int dtype_b, const float* lse_b,
                     int64_t rows, void* out, int dtype_out, float* lse_out,
                     void* stream);

/*
 * mla_merge_states_n -- the [DSMLA] 4.3 merge of `pieces` states per row in
 * one pass, for the partial states of key ranges attended separately. By the
 * merge identity this equals any order of pairwise mla_merge_states calls.
 *
 * Piece p's states: outs[(p * rows + r) * 128 + d] (dtype_in), lses[p * rows + r].
 *   m = max_p lse_p; w_p = e^{lse_p - m} (0 for lse_p = -inf);
 *   out[r * 128 + d] = sum_p w_p outs_p[r][d] / sum_p w_p; lse_out[r] = m + ln sum_p w_p.
 * Pieces at -inf contribute nothing (their out values are loaded but ignored,
 * whatever they hold, so all pieces * rows states must be readable memory);
 * all at -inf gives out = 0, lse = -inf. pieces >= 1. out and lse_out may be piece 0's
 * states (same layout); any other overlap is undefined. dtype_in, dtype_out:
 * MLA_DTYPE_BF16 or MLA_DTYPE_FP32; state pointers 16-byte aligned.
 */
int mla_merge_states_n(const void* outs, int dtype_in, const float* lses, int pieces, int64_t rows,
                       void* out, int dtype_out, float* lse_out, void* stream);

/*
 * mla_merge_states_sets -- up to MLA_MERGE_MAX_SETS independent
 * mla_merge_states_n merges in one launch (for example the Global heads'
 * and the Local rows' partial states of a head-partitioned reuse step), each
 * set with its own pieces, rows and pointers as there, and one dtype pair for
 * all. Every set is checked as mla_merge_states_n checks its arguments;
 * sets with rows = 0 are skipped. The sets must not overlap one another.
 */
#define MLA_MERGE_MAX_SETS 4
typedef struct MlaMergeSet {
  const void* outs;     /* pieces * rows states, dtype_in */
  const float* lses;    /* pieces * rows */
  int pieces;           /* >= 1 */
  int64_t rows;
  void* out;            /* rows states, dtype_out */
  float* lse_out;       /* rows */
} MlaMergeSet;
int mla_merge_states_sets(const MlaMergeSet* sets, int n_sets, int dtype_in, int dtype_out, void* stream);

/*
 * mla_rope_relocate_q -- [REDKNOT] Abstract and section 2 (query-side RoPE
 * relocation): for every row r < T and head h < H, the rope part
 * q[r * q_row_stride + h * 192 + 128 + (0..63)] is rotated by the angle
 * -delta * rope_base^(-2k/64) for pair k (pairing selects which elements form
 * pair k), moving a query at request position p to position p - delta, the
 * canonical frame of a document placed at request offset delta. The 32
 * cos/sin values are computed on the host in fp64 and applied in fp32; the
 * result is rounded to bf16 and written to q_out (same layout and stride).
 * q_out may equal q_in (in place); otherwise the nope part (elements
 * 0..127 of each head) is copied unchanged.
 */
int mla_rope_relocate_q(const void* q_in, void* q_out, int64_t q_row_stride, int T, int H,
                        int64_t delta, double rope_base, int pairing, void* stream);

/*
 * mla_head_partition_merge -- [REDKNOT] sections 1-3 (Equation 4): Local
 * rows come from the artifact except protected rows, which are replaced by
 * their recomputation (not added); Local and Global head outputs go through
 * their slices of the first output projection, add, and pass through the
 * one shared second projection:
 *   O_L[r] = r in prot_rows ? rec_out[index of r] : art_out[r]
 *   z = O_L . W_aL + O_G . W_aG      (bf16 [T][d_mid], fp32 accumulate)
 *   y = z . W_b                      (bf16 [T][d_model])
 *   art_out   device bf16 [T][HL][128];  rec_out bf16 [P][HL][128];
 *   prot_rows device int32 [P], strictly increasing, each in [0, T) (not
 *             checked: the device cannot be read here; out of order, a
 *             protected row may take its artifact row instead, and no access
 *             leaves the given arrays either way);
 *   glob_out  device bf16 [T][HG][128];
 *   wa_t      device bf16 [d_mid][(HL+HG)*128]: [W_aL ; W_aG] stacked along
 *             K (Local rows first) and packed by mla_pack_weight_t;
 *   wb_t      device bf16 [d_model][d_mid]: W_b packed by mla_pack_weight_t;
 *   z         device bf16 [T][d_mid], caller-owned workspace.
 */
int mla_head_partition_merge(const void* art_out, const void* rec_out,
                             const int32_t* prot_rows, int P, const void* glob_out,
                             const void* wa_t, const void* wb_t, int T, int HL, int HG,
                             int d_mid, int d_model, void* z, void* y, void* stream);

/*
 * mla_head_partition_merge_noalloc -- mla_head_partition_merge without the z
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the intermediate z lives in a scratch array inside the
 * library, 8 MiB per device (T * d_mid <= 4194304 bf16 elements; larger
 * calls return MLA_ERR_INVALID_ARG and enqueue nothing). The array is
 * loaded with the library on each device it runs on and held until the
 * process ends; its device address is taken on the first call on a device
 * (no allocation). Every call on one device shares that device's array:
 * calls that overlap on one device (several streams, several threads) race
 * and must be ordered by the caller. z is fully written before it is read,
 * so nothing needs clearing between calls. Arguments, results and errors
 * otherwise as mla_head_partition_merge; MLA_ERR_LAUNCH if the scratch
 * array's address cannot be obtained.
 */
int mla_head_partition_merge_noalloc(const void* art_out, const void* rec_out,
                                     const int32_t* prot_rows, int P, const void* glob_out,
                                     const void* wa_t, const void* wb_t, int T, int HL, int HG,
                                     int d_mid, int d_model, void* y, void* stream);

/*
 * Validation of an offline Local-head artifact before it is reused
 * ([REDKNOT] section 2, "Canonical offline artifacts": each document is
 * processed alone at canonical position zero and its Local-head results are
 * kept; reuse falls back to full recomputation when validation finds missing
 * layers, a token or profile mismatch or a stale generation). The binding of
 * tensor-parallel geometry and the agreement between ranks are not checked
 * here (one device). Host-only functions: no device memory, no stream.
 *
 * mla_artifact_meta describes an artifact (as built) or what a request
 * needs (as served). All fields are plain values:
 *   generation   version of the document's content the artifact was built
 *                from; the request's current version must be equal;
 *   token_hash   mla_token_hash of the document's token ids;
 *   n_tokens     document length in tokens;
 *   n_heads, n_local
 *                logical heads and Local heads (heads 0..n_local-1);
 *   d_c, d_rope, d_nope, d_v
 *                latent, rope, per-head key and value widths;
 *   rope_base    RoPE base of the query/key rotation;
 *   n_layers     reusable layers of the profile (<= 64);
 *   layer_mask   bit l set: layer l's results are present. The request's
 *                value lists the layers it needs.
 */
typedef struct mla_artifact_meta {
  uint64_t generation;
  uint64_t token_hash;
  int64_t n_tokens;
  int32_t n_heads;
  int32_t n_local;
  int32_t d_c;
  int32_t d_rope;
  int32_t d_nope;
  int32_t d_v;
  double rope_base;
  int32_t n_layers;
  int32_t reserved;
  uint64_t layer_mask;
} mla_artifact_meta;

typedef enum {
  MLA_ARTIFACT_VALID = 0,
  MLA_ARTIFACT_MISSING_LAYER = 1,    /* a needed layer is absent            */
  MLA_ARTIFACT_TOKEN_MISMATCH = 2,   /* length or token hash differs        */
  MLA_ARTIFACT_PROFILE_MISMATCH = 3, /* heads, Local split, widths, rope, layer count */
  MLA_ARTIFACT_STALE = 4             /* generation differs                  */
} mla_artifact_reason;

/*
 * mla_token_hash -- 64-bit FNV-1a (Fowler-Noll-Vo, offset basis
 * 0xcbf29ce484222325, prime 0x100000001b3) over the n token ids, each taken
 * as its 4 little-endian bytes. tokens: host int32 [n] (NULL allowed when
 * n == 0). Returns the hash (the offset basis for n == 0).
 */
uint64_t mla_token_hash(const int32_t* tokens, int64_t n);

/*
 * mla_artifact_check -- compares an artifact's description with the
 * request's and writes the first failing check to *reason, in this order:
 * missing layer, token mismatch, profile mismatch, stale generation; else
 * MLA_ARTIFACT_VALID. Returns MLA_OK, or MLA_ERR_INVALID_ARG for a null
 * pointer or a layer count outside 0..64 (then *reason is not written).
 * The caller falls back to full recomputation of the Local heads on any
 * reason other than MLA_ARTIFACT_VALID, before launching the reuse path.
 */
int mla_artifact_check(const mla_artifact_meta* artifact, const mla_artifact_meta* request, int* reason);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
