// gdn_scan.hip -- Gated DeltaNet recurrence over a prompt, state resident in registers.
//
// "Optimizing On-Device Inference for Apple Silicon", section "Keep recurrent state on chip":
// the state matrix of a head is split by rows over groups of lanes, loaded into registers
// once, carried through the whole scan and written back only at the end; partial results
// are exchanged between lanes, not through shared memory; state and gate are fp32, queries
// and keys bf16. The recurrence (the gated delta rule):
//     S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,   o_t = S_t q_t.
// Row i of S evolves on its own given (q_t, k_t, v_t[i], alpha_t, beta_t):
//     b = S_i . k_t,  a = S_i . q_t        (old state)
//     c = beta (v_t[i] - alpha b)
//     o_t[i] = alpha a + c (k_t . q_t)     (= S_i,new . q_t)
//     S_i <- alpha S_i + c k_t
//
// gfx950 mapping: one state row per row of 16 lanes (8 fp32 values per lane, d_k = 128), so
// both dot products reduce with four DPP steps inside the row; a wave holds 4 rows, a
// workgroup 16, and the grid (d_v / 16, value heads) is one workgroup per CU for the model's
// 32 heads. Tokens are staged 64 at a time in LDS (q and k widened to fp32, k . q formed
// once per token for all rows); the next block's loads are in flight in registers while the
// current block is scanned.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kGdnD = 128;      // d_k = d_v
constexpr int kGdnChunk = 64;   // tokens staged per block
constexpr int kGdnRows = 16;    // state rows per workgroup

MOE_DEV float row16_sum_g(float v) {
  v = xor_sum<8>(v);
  v = xor_sum<4>(v);
  v = xor_sum<2>(v);
  return xor_sum<1>(v);
}
}  // namespace

__global__ __launch_bounds__(256, 1) void k_gdn_scan(GdnArgs a) {
  constexpr int D = kGdnD, C = kGdnChunk, R = kGdnRows;
  const int j = blockIdx.y, i0 = blockIdx.x * R;
  const int kh = j / (a.n_v / a.n_k);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int rl = wave * 4 + g;  // this lane group's row inside the workgroup

  __shared__ __attribute__((aligned(16))) float sK[C][D];
  __shared__ __attribute__((aligned(16))) float sQ[C][D];
  __shared__ float sV[C][R];
  __shared__ float sA[C], sB[C], sKQ[C];
  __shared__ __attribute__((aligned(16))) uint16_t sO[C][R];

  // the row's state, 8 values at d = 8 l16 .. +8
  float *srow = a.state + ((size_t)j * D + i0 + rl) * D + 8 * l16;
  float s[8];
  {
    const float4 x = *reinterpret_cast<const float4 *>(srow);
    const float4 y = *reinterpret_cast<const float4 *>(srow + 4);
    s[0] = x.x; s[1] = x.y; s[2] = x.z; s[3] = x.w;
    s[4] = y.x; s[5] = y.y; s[6] = y.z; s[7] = y.w;
  }

  // staging registers of one block: q and k (4 x 16 bytes each per thread), the block's v
  // slice (threads 0..127) or alpha / beta (threads 128..255)
  uint4 rq[4], rk[4], rv;
  float rab = 0.f;
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + 256 * i, tt = f >> 4, part = f & 15;
      const int64_t t = t0 + tt < a.T ? t0 + tt : a.T - 1;
      const size_t off = ((size_t)t * a.n_k + kh) * D + 8 * part;
      rq[i] = *reinterpret_cast<const uint4 *>(a.q + off);
      rk[i] = *reinterpret_cast<const uint4 *>(a.k + off);
    }
    if (tid < 128) {
      const int tt = tid >> 1;
      const int64_t t = t0 + tt < a.T ? t0 + tt : a.T - 1;
      rv = *reinterpret_cast<const uint4 *>(a.v + ((size_t)t * a.n_v + j) * D + i0 + 8 * (tid & 1));
    } else {
      const int tt = (tid - 128) & 63;
      const int64_t t = t0 + tt < a.T ? t0 + tt : a.T - 1;
      rab = (tid < 192 ? a.alpha : a.beta)[(size_t)t * a.n_v + j];
    }
  };
  auto widen = [](uint4 u, float *dst) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float4 lo, hi;
    lo.x = bf16lo(w[0]); lo.y = bf16hi(w[0]); lo.z = bf16lo(w[1]); lo.w = bf16hi(w[1]);
    hi.x = bf16lo(w[2]); hi.y = bf16hi(w[2]); hi.z = bf16lo(w[3]); hi.w = bf16hi(w[3]);
    *reinterpret_cast<float4 *>(dst) = lo;
    *reinterpret_cast<float4 *>(dst + 4) = hi;
  };

  const int64_t nch = (a.T + C - 1) / C;
  fetch(0);
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t t0 = c * C;
    const int nt = (int)(a.T - t0 < C ? a.T - t0 : C);
    __syncthreads();  // the previous block's scan and output copy are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + 256 * i, tt = f >> 4, part = f & 15;
      widen(rq[i], &sQ[tt][8 * part]);
      widen(rk[i], &sK[tt][8 * part]);
    }
    if (tid < 128) {
      float tmp[8];
      widen(rv, tmp);
#pragma unroll
      for (int e = 0; e < 8; ++e) sV[tid >> 1][8 * (tid & 1) + e] = tmp[e];
    } else if (tid < 192) {
      sA[tid - 128] = rab;
    } else {
      sB[tid - 192] = rab;
    }
    __syncthreads();
    {
      // k . q of every token of the block: four threads per token, 32 values each
      const int tt = tid >> 2, part = tid & 3;
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) p = __builtin_fmaf(sK[tt][32 * part + e], sQ[tt][32 * part + e], p);
      p = xor_sum<1>(p);
      p = xor_sum<2>(p);
      if (part == 0) sKQ[tt] = p;
    }
    __syncthreads();
    if (c + 1 < nch) fetch(t0 + C);  // in flight while this block is scanned

#pragma unroll 2
    for (int tt = 0; tt < nt; ++tt) {
      const float4 k0 = *reinterpret_cast<const float4 *>(&sK[tt][8 * l16]);
      const float4 k1 = *reinterpret_cast<const float4 *>(&sK[tt][8 * l16 + 4]);
      const float4 q0 = *reinterpret_cast<const float4 *>(&sQ[tt][8 * l16]);
      const float4 q1 = *reinterpret_cast<const float4 *>(&sQ[tt][8 * l16 + 4]);
      const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      float pb0 = s[0] * kv[0], pb1 = s[1] * kv[1], pa0 = s[0] * qv[0], pa1 = s[1] * qv[1];
#pragma unroll
      for (int e = 2; e < 8; e += 2) {
        pb0 = __builtin_fmaf(s[e], kv[e], pb0);
        pb1 = __builtin_fmaf(s[e + 1], kv[e + 1], pb1);
        pa0 = __builtin_fmaf(s[e], qv[e], pa0);
        pa1 = __builtin_fmaf(s[e + 1], qv[e + 1], pa1);
      }
      const float b = row16_sum_g(pb0 + pb1);
      const float av = row16_sum_g(pa0 + pa1);
      const float al = sA[tt], be = sB[tt];
      const float cc = be * (sV[tt][rl] - al * b);
      const float o = __builtin_fmaf(al, av, cc * sKQ[tt]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = __builtin_fmaf(cc, kv[e], al * s[e]);
      if (l16 == 0) sO[tt][rl] = f32_to_bf16(o);
    }
    __syncthreads();
    // the block's outputs: per token, this workgroup's 16 rows are 32 contiguous bytes
    if (tid < 2 * nt) {
      const int tt = tid >> 1, h = tid & 1;
      *reinterpret_cast<uint4 *>(a.out + ((size_t)(t0 + tt) * a.n_v + j) * D + i0 + 8 * h) =
          *reinterpret_cast<const uint4 *>(&sO[tt][8 * h]);
    }
  }
  *reinterpret_cast<float4 *>(srow) = float4{s[0], s[1], s[2], s[3]};
  *reinterpret_cast<float4 *>(srow + 4) = float4{s[4], s[5], s[6], s[7]};
}

bool gdn_supported(int n_k, int n_v, int d_k, int d_v) {
  return n_k > 0 && n_v > 0 && n_v % n_k == 0 && d_k == kGdnD && d_v == kGdnD;
}

hipError_t launch_gdn_scan(const GdnArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_gdn_scan", k_gdn_scan, dim3(kGdnD / kGdnRows, (unsigned)a.n_v), dim3(256), 0, s,
             a);
  return hipSuccess;
}

}  // namespace moe
