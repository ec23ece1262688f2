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
