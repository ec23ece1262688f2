// Block-table gather of packed latent records (DeepSeek MLA -- Prefix Cache
// and Chunked Prefill, section 4.4 step 1; 64-token blocks per "PagedAttention
// assumed MHA", section "Block size is not a tuning knob here").
//
// HBM-bound copy. A token record is 1152 bytes = 72 vectors of 16 bytes; the
// chunk's records form one stream of vectors. A workgroup moves kVPT * 256
// consecutive vectors, thread i the vectors i, i + 256, ... of that range, so
// every wavefront instruction reads and writes 1 KB of consecutive bytes (a
// cache block holds its 64 records contiguously), and each thread issues all
// its loads before its stores (kVPT loads in flight). fp8 cache: vectors
// 0..63 of a record are 8 E4M3FN codes each (8 bytes in, 16 bytes of bf16
// out), vectors 64..71 copy the bf16 rope key.
#include "mla_internal.h"

namespace {

constexpr int kVecPerTok = kDlat * 2 / 16;   // 72
constexpr int kThreads = 256;
constexpr int kVPT = 4;                      // vectors per thread

template <bool kFp8>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint8_t* __restrict__ pool, int num_blocks, const int32_t* __restrict__ bt,
    int64_t bt_stride, const int32_t* __restrict__ cstart, const int32_t* __restrict__ clen,
    const int32_t* __restrict__ cu_out, uint16_t* __restrict__ out, int32_t* status) {
  const int b = blockIdx.y;
  const int len = clen[b];
  const int start = cstart[b];
  const int64_t obase = cu_out[b];
  const int64_t nvec = (int64_t)len * kVecPerTok;
  const int64_t g0 = (int64_t)blockIdx.x * (kThreads * kVPT) + threadIdx.x;
  if (g0 >= nvec) return;
  u32x4 val[kVPT];
#pragma unroll
  for (int k = 0; k < kVPT; ++k) {
    val[k] = u32x4{0u, 0u, 0u, 0u};
    const int64_t g = g0 + k * kThreads;
    if (g >= nvec) continue;
    const int i = (int)(g / kVecPerTok);
    const int v = (int)(g - (int64_t)i * kVecPerTok);
    const int t = start + i;
    const int lb = t >> 6;
    const int slot = t & 63;
    const int blk = (t >= 0 && lb < bt_stride) ? bt[(int64_t)b * bt_stride + lb] : -1;
    if (blk < 0 || blk >= num_blocks) {
      if (status) status[0] = MLA_ERR_OUT_OF_RANGE;   // the vector is written as zeros
    } else if (!kFp8) {
      const u32x4* src = reinterpret_cast<const u32x4*>(pool + ((int64_t)blk * kBlock + slot) * (kDlat * 2));
      val[k] = __builtin_nontemporal_load(src + v);
    } else {
      const uint8_t* base = pool + (int64_t)blk * kFp8BlockBytes;
      if (v < 64) {
        const u32x2 codes = *reinterpret_cast<const u32x2*>(base + slot * kDc + v * 8);
        const float sc = *reinterpret_cast<const float*>(base + kFp8ScaleOff + slot * 4);
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t c = ((j < 4 ? codes.x : codes.y) >> (8 * (j & 3))) & 0xffu;
          f[j] = e4m3fn_to_f32(c) * sc;
        }
        val[k] = u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                       pack_bf16x2(f[6], f[7])};
      } else {
        val[k] = *reinterpret_cast<const u32x4*>(base + kFp8RopeOff + slot * (kDrope * 2) + (v - 64) * 16);
      }
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + obase * kDlat);
#pragma unroll
  for (int k = 0; k < kVPT; ++k) {
    const int64_t g = g0 + k * kThreads;
    if (g < nvec) dst[g] = val[k];
  }
}

}  // namespace

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
  const int64_t gx = ((int64_t)max_len * kVecPerTok + kThreads * kVPT - 1) / (kThreads * kVPT);
  MLA_REQUIRE(gx < (int64_t)1 << 31, MLA_ERR_INVALID_ARG, "mla_gather_context: max_len too large");
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
