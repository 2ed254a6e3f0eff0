// probe.hip -- a measurement aid, not part of the method: the fp32
// matrix-core throughput a pure v_mfma_f32_32x32x2_f32 loop reaches on this
// GPU, the practical ceiling against which the conv kernels' fractions of
// the 157.3 TFLOP/s specification can also be read.
//
// Every wavefront runs `iters` rounds of 8 independent accumulator chains
// (the conv kernels' wave tile is 8 MFMA blocks too), on constant operands
// (A = B = 1), with no memory traffic; each lane then writes the sum of its
// 128 accumulator elements.  Each MFMA adds 2 (K = 2) to every element, so
// every output is exactly 256 * iters (below 2^24 for iters < 65536).
#include <hip/hip_runtime.h>

#include "dispatch.hpp"

namespace x3 {

typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_probe_kernel(float* out, int iters) {
  probe_f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(1.0f, 1.0f, acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace x3

namespace x3i {

x3_status launch_mfma_probe(float* out, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(x3::mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     out, iters);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(X3_EHIP, "probe kernel launch failed: %s", hipGetErrorString(e));
  return X3_OK;
}

}  // namespace x3i
