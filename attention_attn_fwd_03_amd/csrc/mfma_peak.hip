// Matrix-core rate probe for the measurement tool (not part of the attention
// path): every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on operands
// held in registers, spread over `chains` independent accumulators, so the
// measured rate is what the matrix cores of this chip sustain under the
// current clock, the ceiling the prefill kernels are held against beside the
// published 2.5 PFLOP/s. With chains = 1 every product waits for the previous
// one's accumulator, which shows the dependent-issue latency.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int C>
__global__ __launch_bounds__(256) void mfma_peak_kernel(const uint32_t* seed, float* out, int iters) {
  const int lane = threadIdx.x & 63;
  // operands from memory, so the compiler cannot fold the products
  uint32_t a0 = seed[lane & 15], b0 = seed[16 + (lane & 15)];
  bf16x8 A, B;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A[i] = __builtin_bit_cast(__bf16, (uint16_t)(a0 + i));
    B[i] = __builtin_bit_cast(__bf16, (uint16_t)(b0 + 3 * i));
  }
  f32x16 acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16 / C; ++k)
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Launch `blocks` workgroups of 256 threads (4 waves), each wave issuing
// iters * 16 MFMAs of 32x32x16 (32768 flops each) over `chains` (1, 2, 4, 8
// or 16) accumulators. seed: 32 uint32 on the device; out: blocks * 256
// floats on the device. Returns 0, -1 for bad arguments, -3 for a launch
// error.
int miattn_probe_mfma_peak(const uint32_t* seed, float* out, int blocks, int iters, int chains, void* stream) {
  if (!seed || !out || blocks <= 0 || iters <= 0) return -1;
  hipStream_t st = (hipStream_t)stream;
  switch (chains) {
    case 1: hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    case 2: hipLaunchKernelGGL(mfma_peak_kernel<2>, dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    case 4: hipLaunchKernelGGL(mfma_peak_kernel<4>, dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    case 8: hipLaunchKernelGGL(mfma_peak_kernel<8>, dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    case 16: hipLaunchKernelGGL(mfma_peak_kernel<16>, dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
