// Block-table gather of packed latent records (DeepSeek MLA -- Prefix Cache
// and Chunked Prefill, section 4.4 step 1; 64-token blocks per "PagedAttention
// assumed MHA", section "Block size is not a tuning knob here").
//
// HBM-bound copy. A workgroup moves the records one request has in one
// 64-token cache block (the part of the block inside the request's token
// range): it reads the block id once, and since a block holds its 64 records
// contiguously (bf16 cache) and the output rows are consecutive, the move is
// one contiguous stream of 16-byte vectors, up to 64 * 72 of them, 18 per
// thread, all loads issued before the stores. fp8 cache: vectors 0..63 of a
// record are 8 E4M3FN codes each (8 bytes in, 16 bytes of bf16 out, decoded
// by the hardware conversion) times the token's scale, vectors 64..71 copy
// the bf16 rope key.
#include "mla_internal.h"

namespace {

constexpr int kVecPerTok = kDlat * 2 / 16;   // 72
constexpr int kThreads = 256;
constexpr int kVPT = kBlock * kVecPerTok / kThreads;   // 18 vectors per thread: one whole block
static_assert(kVPT * kThreads == kBlock * kVecPerTok, "a workgroup moves one block");
constexpr int kFp8CodeVPT = kBlock * kDc / 16 / kThreads;        // 8 16-code vectors per thread
constexpr int kFp8RopeVPT = kBlock * kDrope * 2 / 16 / kThreads;  // 2 rope vectors per thread
static_assert(kFp8CodeVPT * kThreads * 16 == kBlock * kDc && kFp8RopeVPT * kThreads * 16 == kBlock * kDrope * 2,
              "fp8 block split");

typedef float f32x2v __attribute__((ext_vector_type(2)));

// 8 E4M3FN codes (two dwords) times the token's scale -> 8 bf16 (four dwords):
// v_cvt_pk_f32_fp8 decodes two OCP E4M3FN codes exactly (the fp8 format of
// gfx950's conversions), the product is one fp32 rounding and
// v_cvt_pk_bf16_f32 rounds to nearest even; NaN (from a NaN code) is written
// as the quiet NaN 0x7FC0, whatever its sign.
__device__ __forceinline__ u32x4 dequant8(u32x2 codes, float sc) {
  float f[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int w = (int)(h ? codes.y : codes.x);
    const f32x2v lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2v hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    f[4 * h + 0] = lo[0] * sc; f[4 * h + 1] = lo[1] * sc;
    f[4 * h + 2] = hi[0] * sc; f[4 * h + 3] = hi[1] * sc;
  }
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t u = cvt_pk_bf16(f[2 * j], f[2 * j + 1]);
    if (__builtin_isnan(f[2 * j])) u = (u & 0xffff0000u) | 0x7fc0u;
    if (__builtin_isnan(f[2 * j + 1])) u = (u & 0x0000ffffu) | 0x7fc00000u;
    o[j] = u;
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

// kRaw (fp8 cache only): the codes are copied as they are into the first
// 512 bytes of each output row and the scales into out_scale; k_rope as
// always at elements 512..575.
template <bool kFp8, bool kRaw = false>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint8_t* __restrict__ pool, int num_blocks, const int32_t* __restrict__ bt,
    int64_t bt_stride, const int32_t* __restrict__ cstart, const int32_t* __restrict__ clen,
    const int32_t* __restrict__ cu_out, uint16_t* __restrict__ out, int32_t* status,
    float* __restrict__ out_scale = nullptr) {
  static_assert(kFp8 || !kRaw, "raw copies are for the fp8 cache");
  const int b = blockIdx.y;
  const int len = clen[b];
  const int start = cstart[b];
  // this workgroup's cache block (the x-th the request's range touches) and
  // the tokens of the range inside it
  const int lb = (start >> 6) + (int)blockIdx.x;
  const int t0 = max(start, lb * kBlock), t1 = min(start + len, lb * kBlock + kBlock);
  if (t1 <= t0) return;
  const int ntok = t1 - t0;
  const int slot0 = t0 & 63;
  const int blk = (t0 >= 0 && lb < bt_stride) ? bt[(int64_t)b * bt_stride + lb] : -1;
  u32x4* dst = reinterpret_cast<u32x4*>(out + ((int64_t)cu_out[b] + (t0 - start)) * kDlat);
  const bool ok = blk >= 0 && blk < num_blocks;
  if (!ok && status && threadIdx.x == 0) status[0] = MLA_ERR_OUT_OF_RANGE;   // written as zeros
  if (!kFp8) {
    // the range's records are one contiguous run in the block
    const int nvec = ntok * kVecPerTok;
    const u32x4* src = reinterpret_cast<const u32x4*>(pool + ((int64_t)blk * kBlock + slot0) * (kDlat * 2));
    u32x4 val[kVPT];
#pragma unroll
    for (int k = 0; k < kVPT; ++k) {
      const int g = threadIdx.x + k * kThreads;
      val[k] = (ok && g < nvec) ? __builtin_nontemporal_load(src + g) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kVPT; ++k) {
      const int g = threadIdx.x + k * kThreads;
      if (g < nvec) dst[g] = val[k];
    }
  } else {
    // The range's codes are one contiguous run of 512 bytes per token: a
    // thread loads 16 codes (one 16-byte vector) per step, all its loads
    // first, and writes the two bf16 vectors each becomes; then the rope
    // keys, 8 vectors per token.
    const uint8_t* base = pool + (int64_t)blk * kFp8BlockBytes;
    const u32x4* csrc = reinterpret_cast<const u32x4*>(base + slot0 * kDc);
    const float* ssrc = reinterpret_cast<const float*>(base + kFp8ScaleOff) + slot0;
    const u32x4* rsrc = reinterpret_cast<const u32x4*>(base + kFp8RopeOff + slot0 * (kDrope * 2));
    u32x4 c16[kFp8CodeVPT], rv[kFp8RopeVPT];
    float sc[kFp8CodeVPT];
#pragma unroll
    for (int k = 0; k < kFp8CodeVPT; ++k) {
      const int cc = threadIdx.x + k * kThreads;    // token cc / 32, codes 16 (cc % 32) .. + 15
      const bool in = ok && (cc >> 5) < ntok;
      c16[k] = in ? __builtin_nontemporal_load(csrc + cc) : u32x4{0u, 0u, 0u, 0u};
      sc[k] = in ? ssrc[cc >> 5] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kFp8RopeVPT; ++k) {
      const int r = threadIdx.x + k * kThreads;      // token r / 8, part r % 8
      rv[k] = (ok && (r >> 3) < ntok) ? rsrc[r] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kFp8CodeVPT; ++k) {
      const int cc = threadIdx.x + k * kThreads;
      const int i = cc >> 5, w = cc & 31;
      if (i >= ntok) continue;
      if constexpr (kRaw) {
        // codes 16 w .. 16 w + 15 of the row's first 512 bytes (zeros for a
        // block outside the pool)
        reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(dst) + i * (kDlat * 2))[w] = c16[k];
        if (w == 0) out_scale[(int64_t)cu_out[b] + (t0 - start) + i] = sc[k];
      } else {
        // zeros stay zeros (a block outside the pool)
        dst[i * kVecPerTok + 2 * w] = ok ? dequant8(u32x2{c16[k].x, c16[k].y}, sc[k]) : u32x4{0u, 0u, 0u, 0u};
        dst[i * kVecPerTok + 2 * w + 1] = ok ? dequant8(u32x2{c16[k].z, c16[k].w}, sc[k]) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int k = 0; k < kFp8RopeVPT; ++k) {
      const int r = threadIdx.x + k * kThreads;
      if ((r >> 3) < ntok) dst[(r >> 3) * kVecPerTok + 64 + (r & 7)] = rv[k];
    }
  }
}

}  // namespace

extern "C" int mla_gather_context_fp8_raw(const void* pool, int num_blocks, const int32_t* block_table,
                                          int64_t bt_stride, const int32_t* chunk_start, const int32_t* chunk_len,
                                          const int32_t* cu_out, int batch, int max_len, void* out_latent,
                                          float* out_scale, int32_t* dev_status, void* stream) {
  mla_begin_call();
  MLA_REQUIRE(batch >= 0 && max_len >= 0, MLA_ERR_INVALID_ARG,
              "mla_gather_context_fp8_raw: batch (%d) and max_len (%d) must be >= 0", batch, max_len);
  if (batch == 0 || max_len == 0) return MLA_OK;
  MLA_REQUIRE(pool && block_table && chunk_start && chunk_len && cu_out && out_latent && out_scale,
              MLA_ERR_INVALID_ARG, "mla_gather_context_fp8_raw: null pointer argument");
  MLA_REQUIRE(num_blocks > 0 && bt_stride > 0, MLA_ERR_INVALID_ARG,
              "mla_gather_context_fp8_raw: num_blocks (%d) and bt_stride (%lld) must be > 0", num_blocks,
              (long long)bt_stride);
  MLA_REQUIRE(mla_aligned16(pool) && mla_aligned16(out_latent) && mla_aligned16(out_scale), MLA_ERR_INVALID_ARG,
              "mla_gather_context_fp8_raw: pool, out_latent and out_scale must be 16-byte aligned");
  MLA_REQUIRE(batch <= 65535, MLA_ERR_INVALID_ARG, "mla_gather_context_fp8_raw: batch (%d) must be <= 65535", batch);
  MLA_REQUIRE((int64_t)max_len + kBlock < (int64_t)1 << 30, MLA_ERR_INVALID_ARG,
              "mla_gather_context_fp8_raw: max_len (%d) too large for one call", max_len);
  const int64_t gx = ((int64_t)max_len + kBlock - 1) / kBlock + 1;
  hipLaunchKernelGGL((gather_kernel<true, true>), dim3((unsigned)gx, (unsigned)batch), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint8_t*>(pool), num_blocks,
                     block_table, bt_stride, chunk_start, chunk_len, cu_out, static_cast<uint16_t*>(out_latent),
                     dev_status, out_scale);
  return mla_check_launch("mla_gather_context_fp8_raw");
}

extern "C" int mla_gather_context(const void* pool, int cache_dtype, int num_blocks,
                                  const int32_t* block_table, int64_t bt_stride,
                                  const int32_t* chunk_start, const int32_t* chunk_len,
                                  const int32_t* cu_out, int batch, int max_len,
                                  void* out_latent, int32_t* dev_status, void* stream) {
  mla_begin_call();
  MLA_REQUIRE(batch >= 0 && max_len >= 0, MLA_ERR_INVALID_ARG,
              "mla_gather_context: batch (%d) and max_len (%d) must be >= 0", batch, max_len);
  if (batch == 0 || max_len == 0) return MLA_OK;
  MLA_REQUIRE(pool && block_table && chunk_start && chunk_len && cu_out && out_latent,
              MLA_ERR_INVALID_ARG, "mla_gather_context: null pointer argument");
  MLA_REQUIRE(num_blocks > 0 && bt_stride > 0, MLA_ERR_INVALID_ARG,
              "mla_gather_context: num_blocks (%d) and bt_stride (%lld) must be > 0",
              num_blocks, (long long)bt_stride);
  MLA_REQUIRE(cache_dtype == MLA_DTYPE_BF16 || cache_dtype == MLA_DTYPE_FP8_E4M3,
              MLA_ERR_UNSUPPORTED, "mla_gather_context: cache dtype %d not supported", cache_dtype);
  MLA_REQUIRE(mla_aligned16(pool) && mla_aligned16(out_latent), MLA_ERR_INVALID_ARG,
              "mla_gather_context: pool and out_latent must be 16-byte aligned");
  MLA_REQUIRE(batch <= 65535, MLA_ERR_INVALID_ARG, "mla_gather_context: batch (%d) must be <= 65535", batch);
  MLA_REQUIRE((int64_t)max_len + kBlock < (int64_t)1 << 30, MLA_ERR_INVALID_ARG,
              "mla_gather_context: max_len (%d) too large for one call", max_len);
  // blocks a range of max_len tokens can touch at any start
  const int64_t gx = ((int64_t)max_len + kBlock - 1) / kBlock + 1;
  dim3 grid((unsigned)gx, (unsigned)batch);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (cache_dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL(gather_kernel<false>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint8_t*>(pool), num_blocks, block_table, bt_stride,
                       chunk_start, chunk_len, cu_out, static_cast<uint16_t*>(out_latent), dev_status);
  else
    hipLaunchKernelGGL(gather_kernel<true>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint8_t*>(pool), num_blocks, block_table, bt_stride,
                       chunk_start, chunk_len, cu_out, static_cast<uint16_t*>(out_latent), dev_status);
  return mla_check_launch("mla_gather_context");
}
