// gemv_tokens.hip -- per-token expert GEMVs on the vector ALUs (batch-1 decode path).
//
// "Optimizing On-Device Inference for Apple Silicon":
//   section "Optimize the one-row weight path" -- one activation row; a wavefront
//   cooperates on each output while its lanes read different parts of the weight row;
//   section "Reduce intermediate and state traffic" -- the two expert input projections
//   are fused with their gated activation, and the output projection is fused with the
//   routing score and the shared-expert result, so temporaries stay in registers.
//
// Only the k selected experts and the shared expert are read. Weight rows are read
// with 16-byte (gate/up) or 8-byte (down) loads from adjacent lanes, so every wave
// load instruction touches one contiguous span of the row.
#include "common.h"
#include "kernels.h"

namespace moe {

// h[t, j, i] = silu(gate_i . x_t) * (up_i . x_t) for expert slot j (k routed + shared).
// One wave per (t, j, i); lane c reads elements [32c, 32c+32) of the gate and up rows.
// Workgroups: blockIdx.x = t * (I/4) + i/4, blockIdx.y = j.
template <bool kInt4>
__global__ __launch_bounds__(256) void k_tok_gateup(TokenArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per_t = a.I / 4;
  const int64_t t = blockIdx.x / per_t;
  const int i = (blockIdx.x % per_t) * 4 + wave;
  const int j = blockIdx.y;
  // ids come from the routing kernels; the clamp only keeps a misused workspace from
  // turning into an out-of-bounds weight read
  const int e = j < a.k ? min(max(a.ids[t * a.k + j], 0), a.E - 1) : a.E;
  const int H = a.H, I = a.I;
  float g = 0.f, u = 0.f;
  if (kInt4) {
    const size_t rg = (size_t)e * 2 * I + i, ru = rg + I;
    const uint8_t *qg = a.wt.w13_q + rg * (H / 2), *qu = a.wt.w13_q + ru * (H / 2);
    const uint16_t *sg = a.wt.w13_s + rg * (H / kGroup), *bg = a.wt.w13_b + rg * (H / kGroup);
    const uint16_t *su = a.wt.w13_s + ru * (H / kGroup), *bu = a.wt.w13_b + ru * (H / kGroup);
    const uint16_t *xt = static_cast<const uint16_t *>(a.x) + t * H;
    for (int c = lane; c < H / 32; c += kWave) {
      const uint4 cg = *reinterpret_cast<const uint4 *>(qg + c * 16);
      const uint4 cu = *reinterpret_cast<const uint4 *>(qu + c * 16);
      const uint4 *xp = reinterpret_cast<const uint4 *>(xt + c * 32);
      const uint4 xw[4] = {xp[0], xp[1], xp[2], xp[3]};
      const uint32_t gw[4] = {cg.x, cg.y, cg.z, cg.w}, uw[4] = {cu.x, cu.y, cu.z, cu.w};
      float qxg = 0.f, qxu = 0.f, sx = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t xs[4] = {xw[wd].x, xw[wd].y, xw[wd].z, xw[wd].w};
        float xv[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          xv[2 * p] = bf16lo(xs[p]);
          xv[2 * p + 1] = bf16hi(xs[p]);
        }
        float q[8], r[8];
        unpack8(gw[wd], q);
        unpack8(uw[wd], r);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          qxg = __builtin_fmaf(q[p], xv[p], qxg);
          qxu = __builtin_fmaf(r[p], xv[p], qxu);
          sx += xv[p];
        }
      }
      // sum_c (s q_c + b) x_c = s sum q x + b sum x  (one group per 64 elements)
      const int grp = c >> 1;
      g += bf16_to_f32(sg[grp]) * qxg + bf16_to_f32(bg[grp]) * sx;
      u += bf16_to_f32(su[grp]) * qxu + bf16_to_f32(bu[grp]) * sx;
    }
  } else {
    const float *wg = a.wt.w13_f + ((size_t)e * 2 * I + i) * H;
    const float *wu = wg + (size_t)I * H;
    const float *xt = static_cast<const float *>(a.x) + t * H;
    for (int c = lane * 4; c < H; c += kWave * 4) {
      const float4 p = *reinterpret_cast<const float4 *>(wg + c);
      const float4 q = *reinterpret_cast<const float4 *>(wu + c);
      const float4 xv = *reinterpret_cast<const float4 *>(xt + c);
      g = __builtin_fmaf(p.x, xv.x, g); g = __builtin_fmaf(p.y, xv.y, g);
      g = __builtin_fmaf(p.z, xv.z, g); g = __builtin_fmaf(p.w, xv.w, g);
      u = __builtin_fmaf(q.x, xv.x, u); u = __builtin_fmaf(q.y, xv.y, u);
      u = __builtin_fmaf(q.z, xv.z, u); u = __builtin_fmaf(q.w, xv.w, u);
    }
  }
  g = wave_sum(g);
  u = wave_sum(u);
  if (lane == 0) a.h[((size_t)t * (a.k + a.S) + j) * I + i] = silu(g) * u;
}

// y[t, r] = sum_j w_j (W2_{e_j} h_j)[r] + (shared W2 h_shared)[r] (+ residual).
// Two output rows per wave (32 lanes each); lane c reads 16 elements of each row.
// Workgroups: blockIdx.x = t * (H/8) + r/8.
template <bool kInt4, bool kBf16>
__global__ __launch_bounds__(256) void k_tok_down(TokenArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per_t = a.H / 8;
  const int64_t t = blockIdx.x / per_t;
  const int row = (blockIdx.x % per_t) * 8 + wave * 2 + (lane >> 5);
  const int sl = lane & 31;
  const int H = a.H, I = a.I, nexp = a.k + a.S;
  float acc = 0.f;
  for (int j = 0; j < nexp; ++j) {
    const int e = j < a.k ? min(max(a.ids[t * a.k + j], 0), a.E - 1) : a.E;
    const float wj = j < a.k ? a.w[t * a.k + j] : 1.0f;
    const float *hj = a.h + ((size_t)t * nexp + j) * I;
    float part = 0.f;
    if (kInt4) {
      const size_t r = (size_t)e * H + row;
      const uint8_t *q = a.wt.w2_q + r * (I / 2);
      const uint16_t *sp = a.wt.w2_s + r * (I / kGroup), *bp = a.wt.w2_b + r * (I / kGroup);
      for (int ch = sl; ch < I / 16; ch += 32) {
        const uint2 cw = *reinterpret_cast<const uint2 *>(q + ch * 8);
        const float4 *hp = reinterpret_cast<const float4 *>(hj + ch * 16);
        const float4 h0 = hp[0], h1 = hp[1], h2 = hp[2], h3 = hp[3];
        const float hv[16] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w,
                              h2.x, h2.y, h2.z, h2.w, h3.x, h3.y, h3.z, h3.w};
        float q0[8], q1[8];
        unpack8(cw.x, q0);
        unpack8(cw.y, q1);
        float qh = 0.f, sh = 0.f;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          qh = __builtin_fmaf(q0[p], hv[p], qh);
          qh = __builtin_fmaf(q1[p], hv[8 + p], qh);
          sh += hv[p] + hv[8 + p];
        }
        const int grp = ch >> 2;
        part += bf16_to_f32(sp[grp]) * qh + bf16_to_f32(bp[grp]) * sh;
      }
    } else {
      const float *wr = a.wt.w2_f + ((size_t)e * H + row) * I;
      for (int c = sl * 4; c < I; c += 128) {
        const float4 p = *reinterpret_cast<const float4 *>(wr + c);
        const float4 hv = *reinterpret_cast<const float4 *>(hj + c);
        part = __builtin_fmaf(p.x, hv.x, part); part = __builtin_fmaf(p.y, hv.y, part);
        part = __builtin_fmaf(p.z, hv.z, part); part = __builtin_fmaf(p.w, hv.w, part);
      }
    }
    acc = __builtin_fmaf(wj, part, acc);
  }
  acc = group_sum<32>(acc);
  if (sl == 0) {
    const size_t o = (size_t)t * H + row;
    if (kBf16) {
      if (a.residual) acc += bf16_to_f32(static_cast<const uint16_t *>(a.residual)[o]);
      static_cast<uint16_t *>(a.y)[o] = f32_to_bf16(acc);
    } else {
      if (a.residual) acc += static_cast<const float *>(a.residual)[o];
      static_cast<float *>(a.y)[o] = acc;
    }
  }
}

hipError_t launch_token_experts(const TokenArgs &a, hipStream_t s) {
  const dim3 g1((unsigned)(a.T * (a.I / 4)), (unsigned)(a.k + a.S));
  const dim3 g2((unsigned)(a.T * (a.H / 8)));
  // int4 weights come with bf16 activations, fp32 weights with fp32 activations
  if (a.int4) {
    MOE_LAUNCH("k_tok_gateup", (k_tok_gateup<true>), g1, dim3(256), 0, s, a);
    MOE_LAUNCH("k_tok_down", (k_tok_down<true, true>), g2, dim3(256), 0, s, a);
  } else {
    MOE_LAUNCH("k_tok_gateup", (k_tok_gateup<false>), g1, dim3(256), 0, s, a);
    MOE_LAUNCH("k_tok_down", (k_tok_down<false, false>), g2, dim3(256), 0, s, a);
  }
  return hipSuccess;
}

}  // namespace moe
