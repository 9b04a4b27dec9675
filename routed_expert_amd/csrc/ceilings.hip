// ceilings.hip -- a dense MFMA loop, the matrix-core ceiling the prefill GEMMs are measured
// against on this GPU at the clock it actually runs under sustained matrix load
// ("Optimizing On-Device Inference for Apple Silicon", section "Limits of further
// optimization": throughput is quoted against the fastest rate measured for the same work,
// besides the nominal peak).
#include "common.h"
#include "kernels.h"

namespace moe {

// Every wave keeps eight independent 32x32 accumulators busy with v_mfma_f32_32x32x16_f16 on
// register operands (no memory traffic in the loop): 512 workgroups of four waves, two per CU
// as in the grouped GEMMs. A thread stores its sum only when it equals a fixed word
// (practically never), so the work cannot be dropped.
__global__ __launch_bounds__(256, 2) void k_mfma_ceiling(int iters, uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  f16x8_t av, bv;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    av[i] = (_Float16)(0.001f * (float)(lane + i));
    bv[i] = (_Float16)(0.002f * (float)(lane - i));
  }
  f32x16_t acc[8] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[q], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[q][r];
  if (__float_as_uint(s) == 0x9E3779B9u) sink[0] = __float_as_uint(s);
}

hipError_t launch_mfma_ceiling(int iters, uint32_t *sink, hipStream_t s) {
  MOE_LAUNCH("k_mfma_ceiling", k_mfma_ceiling, dim3(kMfmaCeilingWG), dim3(256), 0, s, iters, sink);
  return hipSuccess;
}

}  // namespace moe
