// attn_decode.hip -- decode attention of one token over a grouped-query KV cache.
//
// "Optimizing On-Device Inference for Apple Silicon", section "Read the attention cache
// efficiently": the query heads that share a key-value head are packed into one
// workgroup, so every cached K and V row is loaded once for all of them ("Pack query heads
// to reuse KV rows"); neighbouring lanes read neighbouring bytes of the cache ("Coalesce
// attention-cache reads"); and the cache is cut into equal blocks that workgroups process
// in parallel, their partial softmax sums merged afterwards ("Switch attention layouts at
// long contexts").
//
// Differences from the page's design, made for gfx950:
//   - One workgroup takes all eight query heads of a KV head (the page packs four per
//     threadgroup, two threadgroups per KV head): the scores of the eight heads are one
//     16 x 16 x 32 MFMA tile (heads as rows, eight of them padding), so packing costs
//     nothing extra here.
//   - The split into blocks is used at every context length: 256 CUs need hundreds of
//     workgroups, so the number of blocks follows the context (up to 512 workgroups),
//     and a 32K-token cache is already 128 blocks of 256 positions per KV head.
//
// Per wave step (32 positions of one KV head):
//   K rows -> MFMA B operands (lane (n, g): 16 bytes of row t0 + n at d = 32 j + 8 g;
//             four lanes read 64 contiguous bytes of a row per load);
//   S = Q K^T on the MFMA units (fp32 accumulation of exact bf16 products);
//   online softmax in the exp2 domain: row maxima over the 16 lanes of an MFMA row (DPP),
//             running maximum m and sum l per head, previous accumulators rescaled;
//   P (fp32) through the wave's own LDS slice; V rows read coalesced (32 lanes x 16 bytes
//             = one 512-byte row, two rows per load) and accumulated in fp32 on the VALU.
// The four waves of a workgroup interleave over 32-position steps and merge in LDS; the
// workgroup stores (m, l, unnormalised accumulator) per query head; k_attn_combine merges
// the blocks and normalises.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kAttnStep = 32;   // positions per wave step
constexpr int kAttnWaves = 4;
constexpr float kNegInf = -__builtin_inff();

MOE_DEV int64_t imin(int64_t x, int64_t y) { return x < y ? x : y; }

// max over the 16 lanes of a row (xor 8 first, so that the rotation by 4 stands for xor 4)
MOE_DEV float row16_max(float v) {
  v = fmaxf(v, __uint_as_float(xor_peer_dpp<8>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(xor_peer_dpp<4>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(xor_peer_dpp<2>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(xor_peer_dpp<1>(__float_as_uint(v))));
}

MOE_DEV float row16_sum(float v) {
  v = xor_sum<8>(v);
  v = xor_sum<4>(v);
  v = xor_sum<2>(v);
  return xor_sum<1>(v);
}
}  // namespace

// Grid (splits, query-head groups of GP heads). D = 256.
template <int GP>
__global__ __launch_bounds__(256, 2) void k_attn_split(AttnArgs a) {
  constexpr int D = 256, NJ = D / 32;
  const int s = blockIdx.x, qgrp = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;      // MFMA row / column lane and k group
  const int c8 = lane & 31, par = lane >> 5;   // V lanes: 8 values at d = 8 c8, position parity
  const int h0 = qgrp * GP, kvh = h0 / a.G;
  const int64_t t_begin = (int64_t)s * a.tps;
  const int64_t t_end = imin(a.ctx, t_begin + a.tps);
  const uint16_t *K = a.k + (size_t)kvh * a.head_stride;
  const uint16_t *V = a.v + (size_t)kvh * a.head_stride;

  __shared__ __attribute__((aligned(16))) float sP[kAttnWaves][kAttnStep][8];
  __shared__ __attribute__((aligned(16))) float sAl[kAttnWaves][8];
  __shared__ float sM[kAttnWaves][8], sL[kAttnWaves][8];
  __shared__ __attribute__((aligned(16))) float sAcc[kAttnWaves][GP][D];

  // A operands: query head h0 + r (rows past GP are zero), d = 32 j + 8 g .. +8
  bf16x8_t qf[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint4 u = r < GP ? *reinterpret_cast<const uint4 *>(a.q + (size_t)(h0 + r) * D + 32 * j + 8 * g)
                           : uint4{0, 0, 0, 0};
    qf[j] = __builtin_bit_cast(bf16x8_t, u);
  }

  float m[4], lsum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = kNegInf;
    lsum[i] = 0.f;
  }
  float acc[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  // K and V rows of the step at t0 (positions past the block repeat its last row and are
  // masked out of the softmax). Every load of a step is issued before any is used; with two
  // waves per SIMD one wave's loads are in flight while the other computes (issuing the
  // next step's loads early measured slower: the prefetch past a block's end adds a
  // memory round trip before the partial sums can be stored).
  uint4 kb[2][NJ], vb[16];
  auto load_k = [&](int64_t t0) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int64_t t = imin(t0 + 16 * hh + r, t_end - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        kb[hh][j] = *reinterpret_cast<const uint4 *>(K + t * D + 32 * j + 8 * g);
    }
  };
  auto load_v = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t t = imin(t0 + 2 * i + par, t_end - 1);
      vb[i] = *reinterpret_cast<const uint4 *>(V + t * D + 8 * c8);
    }
  };
  for (int64_t t0 = t_begin + wave * kAttnStep; t0 < t_end; t0 += kAttnWaves * kAttnStep) {
    load_k(t0);
    load_v(t0);
    // scores of positions t0 + r (c0) and t0 + 16 + r (c1) for heads 4 g + i
    f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[j], __builtin_bit_cast(bf16x8_t, kb[0][j]),
                                                   c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[j], __builtin_bit_cast(bf16x8_t, kb[1][j]),
                                                   c1, 0, 0, 0);
    }
    const bool ok0 = t0 + r < t_end, ok1 = t0 + 16 + r < t_end;
    float p0[4], p1[4], al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s0 = ok0 ? c0[i] * a.scale_log2 : kNegInf;
      const float s1 = ok1 ? c1[i] * a.scale_log2 : kNegInf;
      const float mn = fmaxf(m[i], row16_max(fmaxf(s0, s1)));
      al[i] = __builtin_amdgcn_exp2f(m[i] - mn);
      p0[i] = __builtin_amdgcn_exp2f(s0 - mn);
      p1[i] = __builtin_amdgcn_exp2f(s1 - mn);
      lsum[i] = lsum[i] * al[i] + (p0[i] + p1[i]);
      m[i] = mn;
    }
    // P [position][head] and the rescale factors of this wave's heads, through its LDS slice
    if (4 * g < GP) {
      *reinterpret_cast<float4 *>(&sP[wave][r][4 * g]) = float4{p0[0], p0[1], p0[2], p0[3]};
      *reinterpret_cast<float4 *>(&sP[wave][16 + r][4 * g]) = float4{p1[0], p1[1], p1[2], p1[3]};
      if (r == 0) *reinterpret_cast<float4 *>(&sAl[wave][4 * g]) = float4{al[0], al[1], al[2], al[3]};
    }
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float f = sAl[wave][h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float *pp = sP[wave][2 * i + par];
      float p[8];
      if constexpr (GP > 4) {
        const float4 x = *reinterpret_cast<const float4 *>(pp);
        const float4 y = *reinterpret_cast<const float4 *>(pp + 4);
        p[0] = x.x; p[1] = x.y; p[2] = x.z; p[3] = x.w;
        p[4] = y.x; p[5] = y.y; p[6] = y.z; p[7] = y.w;
      } else {
        const float4 x = *reinterpret_cast<const float4 *>(pp);
        p[0] = x.x; p[1] = x.y; p[2] = x.z; p[3] = x.w;
      }
      const uint32_t w4[4] = {vb[i].x, vb[i].y, vb[i].z, vb[i].w};
      float v8[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v8[2 * e] = bf16lo(w4[e]);
        v8[2 * e + 1] = bf16hi(w4[e]);
      }
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(p[h], v8[e], acc[h][e]);
    }
    wave_lds_sync();  // the slice is rewritten by the next step
  }

  // this wave's totals: l over the 16 position lanes of a row, accumulators over parities
#pragma unroll
  for (int i = 0; i < 4; ++i) lsum[i] = row16_sum(lsum[i]);
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = xor_sum<32>(acc[h][e]);
  if (r == 0 && 4 * g < GP) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g + i < GP) {
        sM[wave][4 * g + i] = m[i];
        sL[wave][4 * g + i] = lsum[i];
      }
  }
  if (par == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      *reinterpret_cast<float4 *>(&sAcc[wave][h][8 * c8]) =
          float4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
      *reinterpret_cast<float4 *>(&sAcc[wave][h][8 * c8 + 4]) =
          float4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
    }
  }
  __syncthreads();
  // merge the four waves (a wave without positions has m = -inf and contributes nothing)
  for (int o = tid; o < GP * D; o += 256) {
    const int h = o / D, d = o % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sM[w][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sM[w][h] - M);
      L = __builtin_fmaf(f, sL[w][h], L);
      A = __builtin_fmaf(f, sAcc[w][h][d], A);
    }
    const size_t row = (size_t)s * a.n_q + h0 + h;
    a.part_acc[row * D + d] = A;
    if (d == 0) {
      a.part_m[row] = M;
      a.part_l[row] = L;
    }
  }
}

// Merge of the blocks: grid (query heads, D / 16), 256 threads. Thread (split lane sl < 64,
// column quad cq < 4) requests the maxima, sums and 16-byte accumulator slices of its
// blocks s = sl + 64 i, i < NI = ceil(blocks / 64), before using any, so the merge costs one
// memory round trip and no load repeats another; the head's maximum M is a wave reduction
// and four LDS words, each block is weighted by 2^(m_s - M), the split lanes are added in a
// fixed order (within the wave, then over the four waves), and out = sum / l in bf16.
template <int NI>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  constexpr int D = 256;
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cq = lane & 3, sl = (wave << 4) | (lane >> 2);
  const int d0 = blockIdx.y * 16 + 4 * cq;
  float ms[NI], ls[NI];
  float4 vs[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int s = min(sl + 64 * i, a.n_split - 1);
    const size_t row = (size_t)s * a.n_q + h;
    ms[i] = a.part_m[row];
    ls[i] = a.part_l[row];
    vs[i] = *reinterpret_cast<const float4 *>(a.part_acc + row * D + d0);
  }
  __shared__ float wmax[4];
  __shared__ __attribute__((aligned(16))) float4 sacc[4][4];
  __shared__ float swl[4];
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < NI; ++i) mx = fmaxf(mx, ms[i]);  // repeats of the last block are harmless
  // lanes of one column quad differ in lane bits 2..5
  mx = fmaxf(mx, __uint_as_float(xor_peer_dpp<8>(__float_as_uint(mx))));
  mx = fmaxf(mx, __uint_as_float(xor_peer_dpp<4>(__float_as_uint(mx))));  // rotation: ok after 8
  {
    const uint32_t u = __float_as_uint(mx);
    const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    mx = fmaxf(__uint_as_float((uint32_t)p16[0]), __uint_as_float((uint32_t)p16[1]));
    const uint32_t w = __float_as_uint(mx);
    const auto p32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    mx = fmaxf(__uint_as_float((uint32_t)p32[0]), __uint_as_float((uint32_t)p32[1]));
  }
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float lp = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float f = sl + 64 * i < a.n_split ? __builtin_amdgcn_exp2f(ms[i] - M) : 0.f;
    lp = __builtin_fmaf(f, ls[i], lp);
    acc.x = __builtin_fmaf(f, vs[i].x, acc.x);
    acc.y = __builtin_fmaf(f, vs[i].y, acc.y);
    acc.z = __builtin_fmaf(f, vs[i].z, acc.z);
    acc.w = __builtin_fmaf(f, vs[i].w, acc.w);
  }
  auto quad_sum = [](float v) {  // over the 16 lanes of one column quad, order 32, 16, 8, 4
    v = xor_sum<32>(v);
    v = xor_sum<16>(v);
    v = xor_sum<8>(v);
    return xor_sum<4>(v);
  };
  acc.x = quad_sum(acc.x);
  acc.y = quad_sum(acc.y);
  acc.z = quad_sum(acc.z);
  acc.w = quad_sum(acc.w);
  lp = quad_sum(lp);
  if (lane < 4) {
    sacc[wave][cq] = acc;
    if (cq == 0) swl[wave] = lp;
  }
  __syncthreads();
  if (tid < 4) {
    float4 t = sacc[0][tid];
    float L = swl[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 u = sacc[w][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
      L += swl[w];
    }
    const float inv = 1.0f / L;
    uint2 o;
    o.x = pack_bf16x2(t.x * inv, t.y * inv);
    o.y = pack_bf16x2(t.z * inv, t.w * inv);
    *reinterpret_cast<uint2 *>(a.out + (size_t)h * D + blockIdx.y * 16 + 4 * tid) = o;
  }
}

bool attn_supported(int n_q, int n_kv, int D) {
  if (n_q <= 0 || n_kv <= 0 || n_q % n_kv || D != 256) return false;
  const int G = n_q / n_kv;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

// Blocks of the cache: about 128 positions each (a multiple of 32), at most enough for 512
// workgroups over the head groups, never an empty block.
void attn_plan(int64_t ctx, int n_groups, int *n_split, int64_t *tps) {
  const int64_t cap = std::max<int64_t>(1, kAttnMaxSlots / n_groups);
  int64_t ns = std::min<int64_t>(cap, (ctx + 127) / 128);
  if (ns < 1) ns = 1;
  int64_t per = (ctx + ns - 1) / ns;
  per = (per + kAttnStep - 1) / kAttnStep * kAttnStep;
  *tps = per;
  *n_split = (int)((ctx + per - 1) / per);
}

hipError_t launch_attn_decode(const AttnArgs &a, int heads_per_group, hipStream_t s) {
  const unsigned ng = (unsigned)(a.n_q / heads_per_group);
  const dim3 grid((unsigned)a.n_split, ng);
  switch (heads_per_group) {
    case 1: MOE_LAUNCH("k_attn_split", k_attn_split<1>, grid, dim3(256), 0, s, a); break;
    case 2: MOE_LAUNCH("k_attn_split", k_attn_split<2>, grid, dim3(256), 0, s, a); break;
    case 4: MOE_LAUNCH("k_attn_split", k_attn_split<4>, grid, dim3(256), 0, s, a); break;
    case 8: MOE_LAUNCH("k_attn_split", k_attn_split<8>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  const dim3 cgrid((unsigned)a.n_q, 256 / 16);
  static_assert(kAttnMaxSlots <= 8 * 64, "k_attn_combine takes at most 8 blocks per lane");
  if (a.n_split <= 64)
    MOE_LAUNCH("k_attn_combine", k_attn_combine<1>, cgrid, dim3(256), 0, s, a);
  else if (a.n_split <= 128)
    MOE_LAUNCH("k_attn_combine", k_attn_combine<2>, cgrid, dim3(256), 0, s, a);
  else if (a.n_split <= 256)
    MOE_LAUNCH("k_attn_combine", k_attn_combine<4>, cgrid, dim3(256), 0, s, a);
  else
    MOE_LAUNCH("k_attn_combine", k_attn_combine<8>, cgrid, dim3(256), 0, s, a);
  return hipSuccess;
}

}  // namespace moe
