// Query-side RoPE relocation (RedKnot-MLA, Abstract and section 2: queries
// are rotated into a document's canonical frame instead of rewriting the
// document's cached latents).
//
// Rotates the 64-wide rope part of every (row, head) query, in place or into
// a second buffer (then the 128-wide nope part is copied alongside). The 32
// rotation angles -delta * base^(-2k/64) are reduced and evaluated on the
// host in fp64 (delta * theta reaches 2^18 rad and more, far beyond where
// fp32 argument reduction is exact) and passed as fp32 cos/sin pairs.
// HBM-bound: 8 lanes own one head's 128-byte rope slice.
#include <math.h>

#include "mla_internal.h"

namespace {

struct RopeTable {
  float c[32];
  float s[32];
};

constexpr int kThreads = 256;

template <bool kHalf>
__global__ __launch_bounds__(kThreads) void rope_kernel(const uint16_t* qin, uint16_t* qout, int64_t row_stride,
                                                         int T, int H, RopeTable tab) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t rh = gid >> 3;
  const int part = (int)(gid & 7);
  if (rh >= (int64_t)T * H) return;
  const int64_t r = rh / H;
  const int h = (int)(rh - r * H);
  const int64_t off = r * row_stride + (int64_t)h * kDqk;
  if (qin != qout) {
    // out of place: the nope part (16 vectors of 16 B) is copied, 2 per lane
    const u32x4* s = reinterpret_cast<const u32x4*>(qin + off);
    u32x4* d = reinterpret_cast<u32x4*>(qout + off);
    d[part * 2] = s[part * 2];
    d[part * 2 + 1] = s[part * 2 + 1];
  }
  const uint16_t* ibase = qin + off + kDnope;
  uint16_t* base = qout + off + kDnope;
  if (!kHalf) {
    // pairs (2k, 2k+1), k = 4*part .. 4*part+3 : 8 consecutive values
    u32x4* p = reinterpret_cast<u32x4*>(base + part * 8);
    u32x4 u = *reinterpret_cast<const u32x4*>(ibase + part * 8);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = part * 4 + j;
      const float x0 = bf16_bits_to_f32(w[j] & 0xffffu), x1 = bf16_bits_to_f32(w[j] >> 16);
      const float y0 = fmaf(x0, tab.c[k], -x1 * tab.s[k]);
      const float y1 = fmaf(x0, tab.s[k], x1 * tab.c[k]);
      w[j] = pack_bf16x2(y0, y1);
    }
    *p = u32x4{w[0], w[1], w[2], w[3]};
  } else {
    // pairs (k, k+32), k = 4*part .. 4*part+3
    u32x2* p0 = reinterpret_cast<u32x2*>(base + part * 4);
    u32x2* p1 = reinterpret_cast<u32x2*>(base + 32 + part * 4);
    const u32x2 a = *reinterpret_cast<const u32x2*>(ibase + part * 4);
    const u32x2 b = *reinterpret_cast<const u32x2*>(ibase + 32 + part * 4);
    float x0[4] = {bf16_bits_to_f32(a.x & 0xffffu), bf16_bits_to_f32(a.x >> 16),
                   bf16_bits_to_f32(a.y & 0xffffu), bf16_bits_to_f32(a.y >> 16)};
    float x1[4] = {bf16_bits_to_f32(b.x & 0xffffu), bf16_bits_to_f32(b.x >> 16),
                   bf16_bits_to_f32(b.y & 0xffffu), bf16_bits_to_f32(b.y >> 16)};
    float y0[4], y1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = part * 4 + j;
      y0[j] = fmaf(x0[j], tab.c[k], -x1[j] * tab.s[k]);
      y1[j] = fmaf(x0[j], tab.s[k], x1[j] * tab.c[k]);
    }
    *p0 = u32x2{pack_bf16x2(y0[0], y0[1]), pack_bf16x2(y0[2], y0[3])};
    *p1 = u32x2{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3])};
  }
}

}  // namespace

extern "C" int mla_rope_relocate_q(const void* q_in, void* q_out, int64_t q_row_stride, int T, int H,
                                   int64_t delta, double rope_base, int pairing, void* stream) {
  mla_begin_call();
  MLA_REQUIRE(T >= 0 && H >= 0, MLA_ERR_INVALID_ARG, "mla_rope_relocate_q: T and H must be >= 0");
  if (T == 0 || H == 0) return MLA_OK;
  MLA_REQUIRE(q_in && q_out, MLA_ERR_INVALID_ARG, "mla_rope_relocate_q: q is null");
  MLA_REQUIRE(mla_aligned16(q_in) && mla_aligned16(q_out) && q_row_stride % 8 == 0 && q_row_stride >= (int64_t)H * kDqk,
              MLA_ERR_INVALID_ARG,
              "mla_rope_relocate_q: q must be 16-byte aligned with row stride (%lld) a multiple of 8 and >= H*192",
              (long long)q_row_stride);
  MLA_REQUIRE(pairing == MLA_ROPE_INTERLEAVED || pairing == MLA_ROPE_HALF, MLA_ERR_UNSUPPORTED,
              "mla_rope_relocate_q: unknown pairing %d", pairing);
  MLA_REQUIRE(rope_base > 1.0 && isfinite(rope_base), MLA_ERR_INVALID_ARG,
              "mla_rope_relocate_q: rope_base must be finite and > 1");
  // 8 lanes per (row, head): the grid has T * H / 32 workgroups, at most 2^31 - 1
  MLA_REQUIRE((int64_t)T * H <= (int64_t)1 << 34, MLA_ERR_INVALID_ARG,
              "mla_rope_relocate_q: T * H (%lld) too large for one call", (long long)T * H);
  RopeTable tab;
  for (int k = 0; k < 32; ++k) {
    const double theta = pow(rope_base, -2.0 * k / 64.0);
    const double phi = -(double)delta * theta;
    tab.c[k] = (float)cos(phi);
    tab.s[k] = (float)sin(phi);
  }
  const int64_t threads = (int64_t)T * H * 8;
  dim3 g((unsigned)((threads + kThreads - 1) / kThreads));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (pairing == MLA_ROPE_INTERLEAVED)
    hipLaunchKernelGGL(rope_kernel<false>, g, dim3(kThreads), 0, s, static_cast<const uint16_t*>(q_in),
                       static_cast<uint16_t*>(q_out), q_row_stride, T, H, tab);
  else
    hipLaunchKernelGGL(rope_kernel<true>, g, dim3(kThreads), 0, s, static_cast<const uint16_t*>(q_in),
                       static_cast<uint16_t*>(q_out), q_row_stride, T, H, tab);
  return mla_check_launch("mla_rope_relocate_q");
}
