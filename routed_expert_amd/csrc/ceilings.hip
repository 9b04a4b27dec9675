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
// as in the grouped GEMMs. The operands decide the rate: at this part's power limit the
// matrix cores clock down in proportion to the bits they switch, so the loop runs either on
// full-mantissa values (hashed per lane into (-1, 1), like the GEMMs' activations and
// dequantised weights) or on low-entropy ones (multiples of 1/2 below 4). A thread stores its
// sum only when it equals a fixed word (practically never), so the work cannot be dropped.
__global__ __launch_bounds__(256, 2) void k_mfma_ceiling(int iters, int low_entropy,
                                                         uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  f16x8_t av, bv;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (low_entropy) {
      av[i] = (_Float16)(0.5f * (float)((lane + i) & 7));
      bv[i] = (_Float16)(0.5f * (float)i);
    } else {
      uint32_t h = (uint32_t)(threadIdx.x * 8 + i + 1) * 2654435761u;
      h ^= h >> 13;
      h *= 0x5bd1e995u;
      h ^= h >> 15;
      av[i] = (_Float16)((float)(h & 0xFFFFu) * (1.0f / 32768.0f) - 1.0f);
      bv[i] = (_Float16)((float)(h >> 16) * (1.0f / 32768.0f) - 1.0f);
    }
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

hipError_t launch_mfma_ceiling(int iters, int low_entropy, uint32_t *sink, hipStream_t s) {
  MOE_LAUNCH("k_mfma_ceiling", k_mfma_ceiling, dim3(kMfmaCeilingWG), dim3(256), 0, s, iters,
             low_entropy, sink);
  return hipSuccess;
}

}  // namespace moe
