// Achievable bf16 matrix-core throughput of the part: every wave issues long
// runs of independent v_mfma_f32_16x16x32_bf16 (eight accumulators, so no
// instruction waits for the previous one's result). A measurement aid for the
// bench, built as its own library; the tree-GDN path does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kAcc = 8;

__global__ void __launch_bounds__(256) k_mfma_loop(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x4 acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kAcc; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kAcc; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the loop alive
}

}  // namespace

extern "C" {

// Enqueues one launch of `blocks` workgroups of 256 threads, each wave doing
// iters x 8 MFMAs of 16x16x32 (16384 flop each). `out` holds blocks * 256
// floats (device). Returns a hipError_t code.
int gdn_probe_mfma(float* out, int blocks, int iters, hipStream_t s) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(256), 0, s, out, iters);
  return (int)hipGetLastError();
}

// Flops one call performs.
double gdn_probe_mfma_flops(int blocks, int iters) {
  return (double)blocks * 4.0 * iters * kAcc * 16384.0;
}

}
