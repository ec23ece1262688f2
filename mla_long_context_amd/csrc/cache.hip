// Cache write path: append new tokens' packed records [c_kv 512 | k_rope 64]
// into the 64-token blocks of a paged cache (PagedAttention assumed MHA,
// section "Position independence beats prefix matching": records are written
// into blocks that are sealed once full; DeepSeek MLA -- Prefix Cache and
// Chunked Prefill, section 2.2: the latent is stored as fp8).
//
// HBM-bound. One wavefront per token: lane l owns c_kv elements 8l..8l+7
// (one 16-byte read); lanes 0..7 also move the 128-byte rope part. The
// record's max |c_kv| is reduced across the wavefront in registers.
//   bf16 cache: the 1152-byte record is copied.
//   fp8 cache:  scale = fp32(max|c_kv|) / 448 (correctly rounded fp32
//               division), code = E4M3FN round-to-nearest-even of
//               clamp(x / scale, +-448) (each division correctly rounded);
//               a record of zeros gets scale 0 and +0 codes. Codes, rope
//               (bf16) and scale go to the block's three regions
//               (codes [64][512] | rope [64][64] bf16 | scale [64] fp32).
#include "mla_internal.h"

namespace {

constexpr int kWaves = 4;   // tokens per workgroup

// E4M3FN code of an fp32 value with |v| <= 448, round to nearest even:
// normal values (1 + m/8) 2^e, e in [-6, 8], exponent field e + 7; below
// 2^-6 the subnormal code m with value m/8 * 2^-6. A mantissa that rounds up
// to 8 carries into the exponent (m = 8 below 2^-6 is the smallest normal,
// code 0x08, so the same integer works).
__device__ __forceinline__ uint32_t e4m3fn_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a < 0x3c800000u) {                       // |v| < 2^-6: subnormal or zero
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);   // exact scaling, RNE
  } else {
    uint32_t e = (a >> 23) - 127u + 7u;        // exponent field
    uint32_t m = (a >> 20) & 7u;               // top 3 mantissa bits
    const uint32_t rest = a & 0xfffffu;        // 20 dropped bits
    if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) { m = 0u; ++e; }
    code = (e << 3) | m;
  }
  return code | sign;
}

// max over the 64 lanes of a non-negative float, in registers: non-negative
// floats order like their bit patterns, so the reduction runs on integers.
// DPP swaps lanes within quads and rotates 16-lane rows; v_permlane16_swap
// and v_permlane32_swap pair rows and halves (each returns the two swapped
// copies, whose max is the pairwise max).
__device__ __forceinline__ float wave_max_nonneg(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x124, 0xF, 0xF, false));   // row_ror 4
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, false));   // row_ror 8
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = max((uint32_t)r16[0], (uint32_t)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  u = max((uint32_t)r32[0], (uint32_t)r32[1]);
  return __uint_as_float(u);
}

template <bool kFp8>
__global__ __launch_bounds__(kWaves * 64) void append_kernel(uint8_t* pool, int num_blocks,
                                                             const int32_t* __restrict__ bt, int64_t bt_stride,
                                                             const int32_t* __restrict__ pos0,
                                                             const int32_t* __restrict__ cu_new,
                                                             const uint16_t* __restrict__ lat, int64_t ld,
                                                             int32_t* status) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int i = blockIdx.x * kWaves + (threadIdx.x >> 6);   // token of request b
  const int n0 = cu_new[b];
  if (i >= cu_new[b + 1] - n0) return;
  const int t = pos0[b] + i;
  // a position outside the request's block-table row, or a block id outside
  // the pool, is reported and its record skipped
  const bool in_row = t >= 0 && (t >> 6) < bt_stride;
  const int blk = in_row ? bt[(int64_t)b * bt_stride + (t >> 6)] : -1;
  const int slot = t & 63;
  if (blk < 0 || blk >= num_blocks) {
    if (status && lane == 0) *status = MLA_ERR_OUT_OF_RANGE;
    return;
  }
  const uint16_t* src = lat + (int64_t)(n0 + i) * ld;
  const u32x4 c = *reinterpret_cast<const u32x4*>(src + lane * 8);          // c_kv 8l..8l+7
  const u32x4 r = lane < 8 ? *reinterpret_cast<const u32x4*>(src + kDc + lane * 8) : u32x4{0u, 0u, 0u, 0u};
  if (!kFp8) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(pool) + ((int64_t)blk * kBlock + slot) * kDlat;
    *reinterpret_cast<u32x4*>(dst + lane * 8) = c;
    if (lane < 8) *reinterpret_cast<u32x4*>(dst + kDc + lane * 8) = r;
    return;
  }
  float x[8];
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
    x[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
  amax = wave_max_nonneg(amax);
  const float scale = __fdiv_rn(amax, 448.f);
  uint32_t lo = 0u, hi = 0u;
  if (scale > 0.f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float y = fminf(fmaxf(__fdiv_rn(x[j], scale), -448.f), 448.f);
      const uint32_t code = e4m3fn_rne(y);
      if (j < 4) lo |= code << (8 * j);
      else hi |= code << (8 * (j - 4));
    }
  }
  uint8_t* base = pool + (int64_t)blk * kFp8BlockBytes;
  *reinterpret_cast<u32x2*>(base + slot * kDc + lane * 8) = u32x2{lo, hi};
  if (lane < 8) *reinterpret_cast<u32x4*>(base + kFp8RopeOff + slot * kDrope * 2 + lane * 16) = r;
  if (lane == 0) *reinterpret_cast<float*>(base + kFp8ScaleOff + slot * 4) = scale;
}

}  // namespace

extern "C" int mla_cache_append(void* pool, int cache_dtype, int num_blocks, const int32_t* block_table,
                                int64_t bt_stride, const int32_t* pos0, const int32_t* cu_new, int batch,
                                int max_new, const void* latent_new, int64_t ld_latent, int32_t* dev_status,
                                void* stream) {
  mla_begin_call();
  MLA_REQUIRE(batch >= 0 && max_new >= 0 && num_blocks >= 0, MLA_ERR_INVALID_ARG,
              "mla_cache_append: batch, max_new and num_blocks must be >= 0");
  if (batch == 0 || max_new == 0) return MLA_OK;
  MLA_REQUIRE(pool && block_table && pos0 && cu_new && latent_new, MLA_ERR_INVALID_ARG,
              "mla_cache_append: null pointer argument");
  MLA_REQUIRE(cache_dtype == MLA_DTYPE_BF16 || cache_dtype == MLA_DTYPE_FP8_E4M3, MLA_ERR_UNSUPPORTED,
              "mla_cache_append: cache dtype %d not supported", cache_dtype);
  MLA_REQUIRE(mla_aligned16(pool) && mla_aligned16(latent_new), MLA_ERR_INVALID_ARG,
              "mla_cache_append: pool and latent must be 16-byte aligned");
  MLA_REQUIRE(ld_latent >= kDlat && ld_latent % 8 == 0, MLA_ERR_INVALID_ARG,
              "mla_cache_append: ld_latent (%lld) must be >= 576 and a multiple of 8", (long long)ld_latent);
  MLA_REQUIRE(bt_stride > 0, MLA_ERR_INVALID_ARG, "mla_cache_append: bt_stride must be > 0");
  MLA_REQUIRE(batch <= 65535, MLA_ERR_INVALID_ARG, "mla_cache_append: batch (%d) must be <= 65535", batch);
  dim3 g((unsigned)((max_new + kWaves - 1) / kWaves), (unsigned)batch);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* lat = static_cast<const uint16_t*>(latent_new);
  uint8_t* p = static_cast<uint8_t*>(pool);
  if (cache_dtype == MLA_DTYPE_FP8_E4M3)
    hipLaunchKernelGGL(append_kernel<true>, g, dim3(kWaves * 64), 0, s, p, num_blocks, block_table, bt_stride,
                       pos0, cu_new, lat, ld_latent, dev_status);
  else
    hipLaunchKernelGGL(append_kernel<false>, g, dim3(kWaves * 64), 0, s, p, num_blocks, block_table, bt_stride,
                       pos0, cu_new, lat, ld_latent, dev_status);
  return mla_check_launch("mla_cache_append");
}
