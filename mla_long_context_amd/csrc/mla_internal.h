// Internal helpers shared by the gfx950 kernels and the C ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

// ---------------------------------------------------------------- geometry
constexpr int kDc = 512;        // compressed latent width
constexpr int kDrope = 64;      // shared rope key width
constexpr int kDlat = 576;      // packed record: c_kv then k_rope
constexpr int kDnope = 128;
constexpr int kDv = 128;
constexpr int kDqk = 192;
constexpr int kBlock = 64;      // tokens per cache block
constexpr int kFp8BlockBytes = kBlock * kDc + kBlock * kDrope * 2 + kBlock * 4;   // 41216
constexpr int kFp8RopeOff = kBlock * kDc;                                          // 32768
constexpr int kFp8ScaleOff = kFp8RopeOff + kBlock * kDrope * 2;                    // 40960

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- global -> LDS DMA
typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte chunk per lane from global memory into LDS at lds + 16 * lane
// (global_load_lds_dwordx4; the LDS base goes through M0). Issued as inline
// assembly so that the compiler's counter bookkeeping ignores it: completion
// is awaited explicitly with wait_vmcnt before the barrier that publishes a
// tile, and before the workgroup ends.
__device__ __forceinline__ void dma16(const void* src, const void* lds) {
  const uint32_t l = (uint32_t)(uintptr_t)(lds_void*)lds;
  // M0 is a reserved register that compiled code of this file does not use
  // otherwise, so setting it here disturbs nothing
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(l) : "memory");
}

// As dma16, with the source split into a wavefront-uniform base (SGPRs) and a
// per-lane 32-bit byte offset: the address arithmetic of a step is then one
// scalar add, and the per-lane offsets are computed once per tile.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, const void* lds) {
  const uint32_t l = (uint32_t)(uintptr_t)(lds_void*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(l)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------- host error state
void mla_set_error(const char* fmt, ...);
void mla_clear_error();
// start of every entry point that launches: clears the message and any
// stale runtime error left by earlier, unrelated calls
void mla_begin_call();
int mla_check_launch(const char* what);
// compute units of the current device (0 if the runtime cannot tell)
int mla_num_cus();

#define MLA_REQUIRE(cond, code, ...)            \
  do {                                          \
    if (!(cond)) {                              \
      mla_set_error(__VA_ARGS__);               \
      return (code);                            \
    }                                           \
  } while (0)

inline bool mla_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------- device numerics
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Hardware round-to-nearest-even fp32 -> bf16 of two values (v_cvt_pk_bf16_f32);
// used where no NaN can occur and bit patterns of NaN do not matter.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// OCP E4M3FN code -> fp32, exact: bias 7, exponent 0 subnormal (m * 2^-9),
// S.1111.111 NaN, no infinities.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xfu;
  const uint32_t m = c & 7u;
  float v = (e == 0) ? (float)m * 0.001953125f
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15u && m == 7u) v = __uint_as_float(0x7fc00000u);
  return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// Which of the 8 XCDs a linear workgroup id is dispatched to, and the
// remapping that gives each XCD a contiguous range of work items, so that
// work sharing the same operands lands in the same L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t lin, uint32_t total) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = total / kXcd, rem = total % kXcd;
  const uint32_t xcd = lin % kXcd, idx = lin / kXcd;
  // XCDs [0, rem) own per+1 items, the others per.
  const uint32_t base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + idx;
}
