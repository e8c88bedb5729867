// Measurement probe, not part of libkvq (built into libkvq_probe.so, loaded only by
// bench.py): the sustained rate of the FP8 matrix instruction the chunked prefill is
// built on -- v_mfma_scale_f32_32x32x64_f8f6f4, 32 x 32 x 64 e4m3 products summed in
// float32, 131,072 flops per wave and instruction -- as a measured second denominator
// beside the published dense FP8 peak.  Each wave runs four independent accumulator
// chains, so the matrix pipeline never waits for a result, and writes its sums out so
// that the work is kept.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* out) {
  const int lane = (int)threadIdx.x % 64;
  // e4m3 codes around 0x30 (0.5): sums grow by ~16 per instruction and stay finite
  const int x = 0x30303030 + (lane & 3);
  const v8i a = {x, x, x, x, x, x, x, x};
  const v8i b = {x + 1, x, x + 1, x, x + 1, x, x + 1, x};
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// blocks workgroups of 256 threads (4 waves), iters x 4 instructions per wave; out holds
// blocks * 256 floats.  0 on success, 1 for bad arguments, 2 for a launch error.
extern "C" int kvq_probe_mfma_rate(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return 1;
  mfma_rate_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
