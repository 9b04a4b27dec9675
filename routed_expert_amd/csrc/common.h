// common.h -- device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kWave = 64;
constexpr int kGroup = 64;        // int4 quantisation group (weights per scale/bias)
constexpr int kRouteBlock = 64;   // tokens per routing block (histogram granularity)
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;
constexpr int kTileM = 128;       // rows of a grouped-GEMM tile

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
MOE_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round to nearest even; gfx950 lowers this to v_cvt_pk_bf16_f32.
MOE_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Round to nearest even fp16 (v_cvt_pk_f16_f32). Values outside the fp16 range
// become +-inf; callers keep operands inside it.
MOE_DEV uint32_t pack_f16x2(float lo, float hi) {
  f16x2_t v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
MOE_DEV uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

MOE_DEV float f16lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
MOE_DEV float f16hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }

// Two bf16 values (one 32-bit word) to two fp16 values; exact inside the fp16 range.
MOE_DEV uint32_t bf16x2_to_f16x2(uint32_t w) { return pack_f16x2(bf16lo(w), bf16hi(w)); }

// The 8 codes held in one 32-bit word, element order: byte0.lo, byte0.hi, byte1.lo, ...
// q[0..7] receive the codes as floats.
MOE_DEV void unpack8(uint32_t w, float q[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  q[0] = (float)(lo & 0xFF);
  q[1] = (float)(hi & 0xFF);
  q[2] = (float)((lo >> 8) & 0xFF);
  q[3] = (float)((hi >> 8) & 0xFF);
  q[4] = (float)((lo >> 16) & 0xFF);
  q[5] = (float)((hi >> 16) & 0xFF);
  q[6] = (float)(lo >> 24);
  q[7] = (float)(hi >> 24);
}

// Dequantise 8 codes to 4 packed fp16 pairs: w = fp16_rne(fma(s, q, b)).
MOE_DEV uint4 dequant8_f16(uint32_t w, float s, float b) {
  float q[8];
  unpack8(w, q);
  uint4 r;
  r.x = pack_f16x2(__builtin_fmaf(s, q[0], b), __builtin_fmaf(s, q[1], b));
  r.y = pack_f16x2(__builtin_fmaf(s, q[2], b), __builtin_fmaf(s, q[3], b));
  r.z = pack_f16x2(__builtin_fmaf(s, q[4], b), __builtin_fmaf(s, q[5], b));
  r.w = pack_f16x2(__builtin_fmaf(s, q[6], b), __builtin_fmaf(s, q[7], b));
  return r;
}

MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
MOE_DEV float group_sum(float v) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

MOE_DEV float silu(float v) { return v / (1.0f + expf(-v)); }

// Coherent (L1-bypassing) load for data written by other workgroups of the same grid.
MOE_DEV float load_coherent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe
