// Calibration for the benchmark (not part of the prefill library): the
// sustained rate of v_mfma_f32_32x32x16_bf16 on this GPU, from independent
// accumulator chains on every SIMD, so that kernel rates can be read against
// what the matrix cores deliver at the clock the GPU holds under load, beside
// the published peak (which assumes the 2.4 GHz peak clock).
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

// each wavefront: 4 independent chains of `iters` products
__global__ __launch_bounds__(256) void mfma_chains(float* out, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (float)i);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;   // keeps the products live
}

// The attention loop's feed pattern, without its data dependences: per
// iteration 24 products on two accumulator chains whose A operand is read
// from LDS (one 1 KB ds_read_b128 per product, read 6 products ahead), or
// taken from registers (kFeed = 0). kValu adds a softmax's worth of
// independent VALU work per 24 products: 32 exponentials, 64 fmas and 32
// maxima. Workgroups of 4 wavefronts with 64 KB of LDS, so at most two
// share a CU.
// A bf16 value with a random sign and mantissa and an exponent in [2^-8, 2)
// from a 32-bit hash: operands whose bits toggle like those of real data.
__device__ __forceinline__ unsigned short rand_bf16(unsigned x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return (unsigned short)((x & 0x807fu) | ((119u + ((x >> 8) & 7u)) << 7));
}

template <int kFeed, bool kValu, bool kRandom = false>
__global__ __launch_bounds__(256) void mfma_fed(float* out, int iters) {
  constexpr int kLds = 65536;
  __shared__ __attribute__((aligned(1024))) unsigned char sm[kLds];
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kLds / 16; i += 256) {
    u32x4 w = {(unsigned)i, 0x3c003c00u, 0u, 0u};
    if (kRandom)
      for (int e = 0; e < 4; ++e) w[e] = rand_bf16(8u * i + 2u * e) | ((unsigned)rand_bf16(8u * i + 2u * e + 1u) << 16);
    reinterpret_cast<u32x4*>(sm)[i] = w;
  }
  __syncthreads();
  f32x16 s0 = {}, s1 = {};
  bf16x8 q[12];
  for (int s = 0; s < 12; ++s)
    for (int i = 0; i < 8; ++i) {
      if (kRandom)
        q[s][i] = __builtin_bit_cast(__bf16, rand_bf16(0x9e3779b9u + 4096u * blockIdx.x + 96u * tid + 8u * s + i));
      else
        q[s][i] = (__bf16)(0.001f * (float)(lane + s + i));
    }
  float v[32];
  for (int i = 0; i < 32; ++i) v[i] = 0.001f * (float)(lane + i);
  for (int it = 0; it < iters; ++it) {
    // the largest offset read is 3*4096 + 63*16 + 31*128 + 23*1024 + 16 =
    // 40816 bytes, inside the array
    unsigned off = wave * 4096 + lane * 16 + (it & 31) * 128;
    asm volatile("" : "+v"(off));
#pragma unroll
    for (int s = 0; s < 24; ++s) {
      const bf16x8 a = kFeed ? *reinterpret_cast<const bf16x8*>(sm + off + s * 1024) : q[(s + 5) % 12];
      if (s & 1) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[s % 12], s1, 0, 0, 0);
      else s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[s % 12], s0, 0, 0, 0);
    }
    if (kFeed) {
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    }
    if (kValu) {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = __builtin_amdgcn_exp2f(fmaf(v[i], 0.999f, -0.001f));
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = fmaf(v[i], 0.5f, v[(i + 1) & 31]);
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = fmaxf(v[i], v[(i + 7) & 31] * 0.25f);
    }
  }
  float r = 0.f;
  for (int i = 0; i < 16; ++i) r += s0[i] + s1[i];
  for (int i = 0; i < 32; ++i) r += v[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

}  // namespace

// Runs `reps` launches of `workgroups` x 4 wavefronts, each wavefront doing
// 4 * iters products of 32 x 32 x 16, and writes the best rate in TFLOP/s to
// *tflops. out: device float buffer of workgroups * 256 elements (caller
// owned). Returns 0, or -1 on bad arguments or a HIP error.
extern "C" int mla_calib_mfma_bf16(float* out, int workgroups, int iters, int reps, double* tflops) {
  if (!out || !tflops || workgroups <= 0 || iters <= 0 || reps <= 0) return -1;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1;
  if (hipEventCreate(&e1) != hipSuccess) return -1;
  double best = 0.0;
  for (int r = 0; r < reps; ++r) {
    hipEventRecord(e0, 0);
    hipLaunchKernelGGL(mfma_chains, dim3(workgroups), dim3(256), 0, 0, out, iters);
    hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) return -1;
    float ms = 0.f;
    hipEventElapsedTime(&ms, e0, e1);
    const double flops = 2.0 * 32 * 32 * 16 * 4.0 * iters * 4.0 * workgroups;
    if (ms > 0.f && flops / ms / 1e9 > best) best = flops / ms / 1e9;
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  *tflops = best;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Runs `reps` launches of mfma_fed (`workgroups` x 4 wavefronts, 24 * iters
// products per wavefront) and writes the best rate in TFLOP/s to *tflops.
// mode 0: A operand from registers; 1: A operand from LDS, 1 KB per product;
// 2: as 1 plus the independent VALU work; 3: as 1 with random operand bits
// (random signs and mantissas, as real data has) instead of near-constant
// ones. exclusive != 0 adds 40 KB of unused dynamic LDS to each workgroup so
// that no two share a CU (one wavefront per SIMD); otherwise two fit in a
// CU's 160 KB. out: device float buffer of workgroups * 256 elements (caller
// owned). Returns 0, or -1 on bad arguments or a HIP error.
extern "C" int mla_calib_mfma_fed(float* out, int workgroups, int mode, int iters, int reps, int exclusive,
                                  double* tflops) {
  if (!out || !tflops || workgroups <= 0 || iters <= 0 || reps <= 0 || mode < 0 || mode > 3) return -1;
  const unsigned dyn = exclusive ? 40u * 1024u : 0u;
  if (exclusive) {
    const void* kerns[4] = {reinterpret_cast<const void*>(&mfma_fed<0, false>),
                            reinterpret_cast<const void*>(&mfma_fed<1, false>),
                            reinterpret_cast<const void*>(&mfma_fed<1, true>),
                            reinterpret_cast<const void*>(&mfma_fed<1, false, true>)};
    if (hipFuncSetAttribute(kerns[mode], hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn) != hipSuccess) return -1;
  }
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1;
  if (hipEventCreate(&e1) != hipSuccess) return -1;
  double best = 0.0;
  for (int r = 0; r < reps; ++r) {
    hipEventRecord(e0, 0);
    if (mode == 0) hipLaunchKernelGGL((mfma_fed<0, false>), dim3(workgroups), dim3(256), dyn, 0, out, iters);
    else if (mode == 1) hipLaunchKernelGGL((mfma_fed<1, false>), dim3(workgroups), dim3(256), dyn, 0, out, iters);
    else if (mode == 2) hipLaunchKernelGGL((mfma_fed<1, true>), dim3(workgroups), dim3(256), dyn, 0, out, iters);
    else hipLaunchKernelGGL((mfma_fed<1, false, true>), dim3(workgroups), dim3(256), dyn, 0, out, iters);
    hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) return -1;
    float ms = 0.f;
    hipEventElapsedTime(&ms, e0, e1);
    const double flops = 2.0 * 32 * 32 * 16 * 24.0 * iters * 4.0 * workgroups;
    if (ms > 0.f && flops / ms / 1e9 > best) best = flops / ms / 1e9;
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  *tflops = best;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
