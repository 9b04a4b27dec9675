// combine.hip -- weighted combine of expert outputs back to token order, and the
// RMSNorm used between stacked layers.
//
// "Optimizing On-Device Inference for Apple Silicon", section "Reduce intermediate
// and state traffic": each expert's output projection is combined with its routing
// score and with the shared-expert result. In the prefill path the down GEMM writes each
// routed slot's output already scaled by its routing weight and the shared expert's
// output after them (slots kT + t), all fp16; this kernel gathers a token's rows in a
// fixed order (shared first, then ascending expert id) and sums them in fp32, so the
// result is deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int64_t t = blockIdx.x;
  const int k = a.k, H = a.H;
  size_t row[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    row[j] = (size_t)a.slot_of[t * k + j] * H;
  }
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    const size_t o = (size_t)t * H + c;
    float acc[8];
    if (a.S) {
      const uint4 v =
          *reinterpret_cast<const uint4 *>(a.out + ((size_t)k * a.T + t) * H + c);
      acc[0] = f16lo(v.x); acc[1] = f16hi(v.x); acc[2] = f16lo(v.y); acc[3] = f16hi(v.y);
      acc[4] = f16lo(v.z); acc[5] = f16hi(v.z); acc[6] = f16lo(v.w); acc[7] = f16hi(v.w);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) break;
      const uint4 v = *reinterpret_cast<const uint4 *>(a.out + row[j] + c);
      acc[0] += f16lo(v.x); acc[1] += f16hi(v.x); acc[2] += f16lo(v.y);
      acc[3] += f16hi(v.y); acc[4] += f16lo(v.z); acc[5] += f16hi(v.z);
      acc[6] += f16lo(v.w); acc[7] += f16hi(v.w);
    }
    if (a.residual) {
      const uint4 v = *reinterpret_cast<const uint4 *>(a.residual + o);
      acc[0] += bf16lo(v.x); acc[1] += bf16hi(v.x); acc[2] += bf16lo(v.y);
      acc[3] += bf16hi(v.y); acc[4] += bf16lo(v.z); acc[5] += bf16hi(v.z);
      acc[6] += bf16lo(v.w); acc[7] += bf16hi(v.w);
    }
    uint4 r;
    r.x = pack_bf16x2(acc[0], acc[1]);
    r.y = pack_bf16x2(acc[2], acc[3]);
    r.z = pack_bf16x2(acc[4], acc[5]);
    r.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4 *>(a.y + o) = r;
  }
}

// out[t] = h[t] / sqrt(mean(h[t]^2) + eps); one workgroup per row, fp32 arithmetic.
// h and out may alias: every element is read and written by the same thread.
template <bool kBf16>
__global__ __launch_bounds__(256) void k_rmsnorm(const void *h, int H, float eps, void *out) {
  __shared__ float part[4];
  const size_t base = (size_t)blockIdx.x * H;
  const int tid = threadIdx.x;
  auto ld = [&](int c) {
    return kBf16 ? bf16_to_f32(static_cast<const uint16_t *>(h)[base + c])
                 : static_cast<const float *>(h)[base + c];
  };
  float ss = 0.f;
  for (int c = tid; c < H; c += 256) {
    const float v = ld(c);
    ss = __builtin_fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float total = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(total / (float)H + eps);
  for (int c = tid; c < H; c += 256) {
    const float v = ld(c) * inv;
    if (kBf16)
      static_cast<uint16_t *>(out)[base + c] = f32_to_bf16(v);
    else
      static_cast<float *>(out)[base + c] = v;
  }
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_combine", k_combine, dim3((unsigned)a.T), dim3(256), 0, s, a);
  return hipSuccess;
}

hipError_t launch_rmsnorm(const void *h, int64_t T, int H, float eps, bool bf16, void *out,
                          hipStream_t s) {
  if (bf16)
    MOE_LAUNCH("k_rmsnorm", k_rmsnorm<true>, dim3((unsigned)T), dim3(256), 0, s, h, H, eps, out);
  else
    MOE_LAUNCH("k_rmsnorm", k_rmsnorm<false>, dim3((unsigned)T), dim3(256), 0, s, h, H, eps,
               out);
  return hipSuccess;
}

}  // namespace moe
