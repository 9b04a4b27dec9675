// combine.hip -- weighted combine of expert outputs back to token order, and the
// RMSNorm used between stacked layers.
//
// "Optimizing On-Device Inference for Apple Silicon", section "Reduce intermediate
// and state traffic": each expert's output projection is combined with its routing
// score and with the shared-expert result. In the prefill path the down GEMM writes each
// routed slot's output already scaled by its routing weight, in fp16. With a shared expert
// the combine runs in the shared expert's down projection (k_shared_down_combine); this
// kernel serves layers without one: it gathers a token's k rows in a fixed order
// (ascending expert id) and sums them in fp32, so the result is deterministic.
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
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
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

// out[t] = h[t] / sqrt(mean(h[t]^2) + eps); one workgroup of 512 threads per row, fp64
// arithmetic rounded once to the output dtype (bf16: round to nearest even from the fp64
// value). Thread t takes elements 4t .. 4t+3 of each 2048-element stretch, the layout of the
// fused decode normalisation, so both give the same bits. h and out may alias: every
// element is read and written by the same thread.
template <bool kBf16>
__global__ __launch_bounds__(512) void k_rmsnorm(const void *h, int H, float eps, void *out) {
  __shared__ double red8[8];
  const size_t base = (size_t)blockIdx.x * H;
  const int tid = threadIdx.x;
  auto ld = [&](int c) {
    return kBf16 ? (double)bf16_to_f32(static_cast<const uint16_t *>(h)[base + c])
                 : (double)static_cast<const float *>(h)[base + c];
  };
  double ss = 0.0;
  for (int c0 = 4 * tid; c0 < H; c0 += 2048)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c0 + i < H) {
        const double v = ld(c0 + i);
        ss = __builtin_fma(v, v, ss);
      }
  const double inv = row_inv_rms_f64(ss, H, (double)eps, red8);
  for (int c0 = 4 * tid; c0 < H; c0 += 2048)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c0 + i < H) {
        const double v = ld(c0 + i) * inv;
        if (kBf16)
          static_cast<uint16_t *>(out)[base + c0 + i] = f64_to_bf16_rne(v);
        else
          static_cast<float *>(out)[base + c0 + i] = (float)v;
      }
}

// The same normalisation for bf16 rows whose H is a multiple of 2048 (at most kNormMaxH): one
// wave per row, four rows per workgroup, with the bits of k_rmsnorm. Lane l stands in for the
// threads l + 64 w (w = 0..7) of k_rmsnorm's 512: each virtual thread's partial is the fma
// chain over its four elements of every 2048-element stretch in index order, each of the eight
// partials goes through the xor butterfly of a wave, and the eight wave totals are added in
// wave order. Every element is read once (four bf16 per 8-byte load, 512 contiguous bytes per
// load instruction) and scaled from registers; h and out may alias.
constexpr int kNormMaxH = 8192;
template <int NS>  // 2048-element stretches per row
__global__ __launch_bounds__(256) void k_rmsnorm_rows(const uint16_t *h, int64_t T, float eps,
                                                      uint16_t *out) {
  constexpr int H = 2048 * NS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= T) return;
  const size_t base = (size_t)row * H + 4 * lane;
  uint2 v[NS][8];
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int w = 0; w < 8; ++w)
      v[j][w] = *reinterpret_cast<const uint2 *>(h + base + 2048 * j + 256 * w);
  double p[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    p[w] = 0.0;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const double e0 = bf16lo(v[j][w].x), e1 = bf16hi(v[j][w].x);
      const double e2 = bf16lo(v[j][w].y), e3 = bf16hi(v[j][w].y);
      p[w] = __builtin_fma(e0, e0, p[w]);
      p[w] = __builtin_fma(e1, e1, p[w]);
      p[w] = __builtin_fma(e2, e2, p[w]);
      p[w] = __builtin_fma(e3, e3, p[w]);
    }
  }
  // the xor butterfly over the wave (32, 16, 8, 4, 2, 1; the pairs of block512_sum_f64),
  // the eight chains side by side: here the crossbar's latency overlaps across the chains,
  // and __shfl_xor measured faster than the DPP form that a single chain prefers
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
    for (int w = 0; w < 8; ++w) p[w] += __shfl_xor(p[w], m, kWave);
  double total = p[0];
#pragma unroll
  for (int w = 1; w < 8; ++w) total += p[w];
  const double inv = 1.0 / sqrt(total / (double)H + (double)eps);
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint2 u = v[j][w];
      const uint32_t lo = (uint32_t)f64_to_bf16_rne((double)bf16lo(u.x) * inv) |
                          ((uint32_t)f64_to_bf16_rne((double)bf16hi(u.x) * inv) << 16);
      const uint32_t hi = (uint32_t)f64_to_bf16_rne((double)bf16lo(u.y) * inv) |
                          ((uint32_t)f64_to_bf16_rne((double)bf16hi(u.y) * inv) << 16);
      *reinterpret_cast<uint2 *>(out + base + 2048 * j + 256 * w) = make_uint2(lo, hi);
    }
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_combine", k_combine, dim3((unsigned)a.T), dim3(256), 0, s, a);
  return hipSuccess;
}

hipError_t launch_rmsnorm(const void *h, int64_t T, int H, float eps, bool bf16, void *out,
                          hipStream_t s) {
  const dim3 g4((unsigned)((T + 3) / 4));
  const uint16_t *hb = static_cast<const uint16_t *>(h);
  uint16_t *ob = static_cast<uint16_t *>(out);
  // the one-wave-per-row kernel loads and stores 8-byte pieces
  const bool rows = bf16 && !(((uintptr_t)h | (uintptr_t)out) & 7);
  if (rows && H == 2048)
    MOE_LAUNCH("k_rmsnorm_rows", k_rmsnorm_rows<1>, g4, dim3(256), 0, s, hb, T, eps, ob);
  else if (rows && H == 4096)
    MOE_LAUNCH("k_rmsnorm_rows", k_rmsnorm_rows<2>, g4, dim3(256), 0, s, hb, T, eps, ob);
  else if (rows && H == 6144)
    MOE_LAUNCH("k_rmsnorm_rows", k_rmsnorm_rows<3>, g4, dim3(256), 0, s, hb, T, eps, ob);
  else if (rows && H == kNormMaxH)
    MOE_LAUNCH("k_rmsnorm_rows", k_rmsnorm_rows<4>, g4, dim3(256), 0, s, hb, T, eps, ob);
  else if (bf16)
    MOE_LAUNCH("k_rmsnorm", k_rmsnorm<true>, dim3((unsigned)T), dim3(512), 0, s, h, H, eps, out);
  else
    MOE_LAUNCH("k_rmsnorm", k_rmsnorm<false>, dim3((unsigned)T), dim3(512), 0, s, h, H, eps,
               out);
  return hipSuccess;
}

}  // namespace moe
