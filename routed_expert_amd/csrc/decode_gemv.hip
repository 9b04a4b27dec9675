// decode_gemv.hip -- batch-1 MoE layer (hidden 2048, intermediate 512, int4 g64) in three
// lean kernels on the vector ALUs.
//
// "Optimizing On-Device Inference for Apple Silicon":
//   section "Decode: minimize the bytes moved per token" -- only the router, the k
//   selected experts and the shared expert are read, each byte once;
//   section "Optimize the one-row weight path" -- row-parallel GEMVs: a wavefront
//   cooperates on one output row while its lanes read adjacent 16-byte pieces of it;
//   section "Overlap independent GPU work" -- the shared expert does not depend on the
//   routing, so its gate/up projection runs next to the router;
//   section "Reduce intermediate and state traffic" -- gate/up are fused with SwiGLU and
//   the output projection with the routing weights and the shared-expert result.
//
// The kernel boundaries are the two device-wide exchanges the layer needs (all router
// logits before the top-k, all of h before the output projection). Inside a HIP graph a
// boundary costs about 1.8 us on MI355X, measured below a grid barrier built on
// device-scope atomics across 256 workgroups (2.4-3.7 us), so no kernel spins.
//
//   A  256 workgroups x 512 threads: workgroup w computes router logit z[w]; waves 0-1
//      compute shared-expert gate/up pairs i = wave*256 + w and store h_shared[i].
//   B  every workgroup runs the top-k on z (same data, same code, same answer) and
//      computes routed gate/up tasks (j, i) = slot and slot + 2048, slot = wave*256 + w.
//      Workgroup 0 stores the ids and weights for C.
//   C  wave computes output row c = wave*256 + w of the down projection over all k+1
//      experts (h staged in LDS), adds the residual and stores y[c].
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int DH = 2048, DI = 512, DWG = 256, DT = 512;
constexpr int kSlots = kMaxTopK + 1;
}  // namespace

// Lane's 32 activations [32*lane, 32*lane+32) of the 2048-element bf16 row.
MOE_DEV void load_x32(const uint16_t *x, int lane, float xv[32]) {
  const uint4 *xp = reinterpret_cast<const uint4 *>(x + lane * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = xp[i];
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      xv[8 * i + 2 * p] = bf16lo(wd[p]);
      xv[8 * i + 2 * p + 1] = bf16hi(wd[p]);
    }
  }
}

// Sum over the lane's 32 codes (16 bytes) times its 32 activations.
MOE_DEV float dot32(const uint4 c, const float x[32]) {
  const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float q[8];
    unpack8(wd[i], q);
#pragma unroll
    for (int p = 0; p < 8; ++p) acc = __builtin_fmaf(q[p], x[8 * i + p], acc);
  }
  return acc;
}

// One gate/up row pair (rows r and r + I of expert e's W13) against the lane's x.
struct RowPair {
  uint4 cg, cu;
  uint16_t sg, bg, su, bu;
};

MOE_DEV RowPair load_pair(const ExpertWeights &wt, int e, int i, int lane) {
  const size_t rg = (size_t)e * 2 * DI + i, ru = rg + DI;
  const int grp = lane >> 1;
  RowPair p;
  p.cg = reinterpret_cast<const uint4 *>(wt.w13_q + rg * (DH / 2))[lane];
  p.cu = reinterpret_cast<const uint4 *>(wt.w13_q + ru * (DH / 2))[lane];
  p.sg = wt.w13_s[rg * (DH / kGroup) + grp];
  p.bg = wt.w13_b[rg * (DH / kGroup) + grp];
  p.su = wt.w13_s[ru * (DH / kGroup) + grp];
  p.bu = wt.w13_b[ru * (DH / kGroup) + grp];
  return p;
}

// silu(gate . x) * (up . x); sum over a group of (s q + b) x = s (q . x) + b (sum x)
MOE_DEV float pair_h(const RowPair &p, const float xv[32], float sx) {
  const float g = wave_sum_dpp(bf16_to_f32(p.sg) * dot32(p.cg, xv) + bf16_to_f32(p.bg) * sx);
  const float u = wave_sum_dpp(bf16_to_f32(p.su) * dot32(p.cu, xv) + bf16_to_f32(p.bu) * sx);
  return silu(g) * u;
}

MOE_DEV float lane_xsum(const float xv[32]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) s += xv[i];
  return s;
}

// Top-k of the E <= 256 router logits using all 8 waves of the workgroup (latency: the
// chain of dependent instructions is what costs time for a single wave). Keys are 64-bit:
// float key high, ~id low, so one unsigned compare orders by (logit desc, id asc).
//   1. wave v ranks elements [32v, 32v+32) among themselves (two lanes per element, 16
//      comparisons each); its k best go to cand[8v ..].
//   2. the 64 candidates are ranked among each other (lane: candidate 8v + l%8 against
//      comparands 8(l/8) .. 8(l/8)+7, partial ranks summed over the 8 lane groups).
//   3. lanes 0..k-1 of wave 0 turn the k winners into ids in ascending order and softmax
//      weights.
// Must be called by all DT threads; results land in s_ids / s_w.
MOE_DEV void block_topk(const float *z, int E, int k, uint64_t *K, uint64_t *cand,
                        int *s_ids, float *s_w) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < 256) {
    const float f = tid < E ? z[tid] : -INFINITY;
    const float g = f != f ? -INFINITY : f;
    K[tid] = tid < E ? ((uint64_t)float_key(g) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)tid)
                     : 0ull;
  }
  if (tid < 64) cand[tid] = 0ull;
  __syncthreads();
  {
    const int e = 32 * wave + (lane & 31), half = lane >> 5;
    const uint64_t mine = K[e];
    const uint64_t *base = K + 32 * wave + 16 * half;
    int r = 0;
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
      const ulonglong2 p = *reinterpret_cast<const ulonglong2 *>(base + q);
      r += (p.x > mine) + (p.y > mine);
    }
    r += __shfl_xor(r, 32, 64);
    if (half == 0 && r < k) cand[8 * wave + r] = mine;
  }
  __syncthreads();
  {
    const int ci = 8 * wave + (lane & 7), seg = lane >> 3;
    const uint64_t mine = cand[ci];
    const uint64_t *base = cand + 8 * seg;
    int r = 0;
#pragma unroll
    for (int q = 0; q < 8; q += 2) {
      const ulonglong2 p = *reinterpret_cast<const ulonglong2 *>(base + q);
      r += (p.x > mine) + (p.y > mine);
    }
    r += __shfl_xor(r, 8, 64);
    r += __shfl_xor(r, 16, 64);
    r += __shfl_xor(r, 32, 64);
    if (seg == 0 && mine != 0ull && r < k) K[r] = mine;  // K reused for the winners
  }
  __syncthreads();
  if (tid < 64) {
    const uint64_t b = tid < k ? K[tid] : 0ull;
    const int id = (int)(0xFFFFFFFFu - (uint32_t)b);
    const float v = key_float((uint32_t)(b >> 32));
    const float top = key_float((uint32_t)(K[0] >> 32));
    const float ex = tid < k ? (top == -INFINITY ? 1.0f : expf(v - top)) : 0.f;
    float den = ex;
    den += __shfl_xor(den, 1, 64);
    den += __shfl_xor(den, 2, 64);
    den += __shfl_xor(den, 4, 64);
    int rk = 0;
    for (int q = 0; q < k; ++q) rk += __shfl(id, q, 64) < id ? 1 : 0;
    if (tid < k) {
      s_ids[rk] = id;
      s_w[rk] = ex / den;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(DT) void k_dec_a(DecodeArgs a) {
  __shared__ float red[DT / 64];
  const int w = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  RowPair sp;
  const bool do_shared = a.S && wave < 2;
  if (do_shared) sp = load_pair(a.wt, a.E, wave * DWG + w, lane);
  if (w < a.E) {
    const float4 wr = reinterpret_cast<const float4 *>(a.router_w + (size_t)w * DH)[tid];
    const uint2 xb = reinterpret_cast<const uint2 *>(a.x)[tid];
    float d = wr.x * bf16lo(xb.x);
    d = __builtin_fmaf(wr.y, bf16hi(xb.x), d);
    d = __builtin_fmaf(wr.z, bf16lo(xb.y), d);
    d = __builtin_fmaf(wr.w, bf16hi(xb.y), d);
    d = wave_sum_dpp(d);
    if (lane == 0) red[wave] = d;
  }
  if (do_shared) {
    float xv[32];
    load_x32(a.x, lane, xv);
    const float hv = pair_h(sp, xv, lane_xsum(xv));
    if (lane == 0) a.h[(size_t)a.k * DI + wave * DWG + w] = hv;
  }
  __syncthreads();
  if (tid == 0 && w < a.E) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < DT / 64; ++i) s += red[i];
    a.z[w] = s + (a.router_b ? a.router_b[w] : 0.f);
  }
}

__global__ __launch_bounds__(DT) void k_dec_b(DecodeArgs a) {
  __shared__ int s_ids[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ __attribute__((aligned(16))) uint64_t s_key[256];
  __shared__ __attribute__((aligned(16))) uint64_t s_cand[64];
  const int w = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float xv[32];
  load_x32(a.x, lane, xv);
  block_topk(a.z, a.E, a.k, s_key, s_cand, s_ids, s_w);
  if (w == 0 && tid < a.k) {
    a.ids_out[tid] = s_ids[tid];
    a.w_out[tid] = s_w[tid];
  }
  const float sx = lane_xsum(xv);
  const int slot = wave * DWG + w;
  const int j0 = slot / DI, j1 = (slot + DWG * DT / 64) / DI;
  const bool t0 = j0 < a.k, t1 = j1 < a.k;
  RowPair p0, p1;
  if (t0) p0 = load_pair(a.wt, s_ids[j0], slot % DI, lane);
  if (t1) p1 = load_pair(a.wt, s_ids[j1], (slot + DWG * DT / 64) % DI, lane);
  if (t0) {
    const float hv = pair_h(p0, xv, sx);
    if (lane == 0) a.h[(size_t)j0 * DI + slot % DI] = hv;
  }
  if (t1) {
    const float hv = pair_h(p1, xv, sx);
    if (lane == 0) a.h[(size_t)j1 * DI + (slot + DWG * DT / 64) % DI] = hv;
  }
}

__global__ __launch_bounds__(DT) void k_dec_c(DecodeArgs a) {
  __shared__ float hs[kSlots * DI];
  __shared__ int s_ids[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int w = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int k = a.k, nslot = a.k + a.S;
  // h of all k+1 experts into LDS (independent of the routing ids)
  float hr[kSlots];
#pragma unroll
  for (int q = 0; q < kSlots; ++q) {
    const int i = tid + q * DT;
    hr[q] = i < nslot * DI ? a.h[i] : 0.f;
  }
  if (tid < k) {
    s_ids[tid] = min(max(a.ids_out[tid], 0), a.E - 1);
    s_w[tid] = a.w_out[tid];
  }
#pragma unroll
  for (int q = 0; q < kSlots; ++q) {
    const int i = tid + q * DT;
    if (i < nslot * DI) hs[i] = hr[q];
  }
  __syncthreads();
  // lane slots s = lane + 64 m: expert slot j = s / 32, 16-element chunk ch = s % 32
  const int c_row = wave * DWG + w;
  uint2 cw[5];
  uint16_t sc[5], bc[5];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int s = lane + 64 * m, j = s >> 5, ch = s & 31;
    if (j < nslot) {
      const int e = j < k ? s_ids[j] : a.E;
      const size_t r = (size_t)e * DH + c_row;
      cw[m] = reinterpret_cast<const uint2 *>(a.wt.w2_q + r * (DI / 2))[ch];
      sc[m] = a.wt.w2_s[r * (DI / kGroup) + (ch >> 2)];
      bc[m] = a.wt.w2_b[r * (DI / kGroup) + (ch >> 2)];
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int s = lane + 64 * m, j = s >> 5, ch = s & 31;
    if (j < nslot) {
      const float *hp = hs + j * DI + ch * 16;
      float q0[8], q1[8];
      unpack8(cw[m].x, q0);
      unpack8(cw[m].y, q1);
      float qh = 0.f, sh = 0.f;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        qh = __builtin_fmaf(q0[p], hp[p], qh);
        qh = __builtin_fmaf(q1[p], hp[8 + p], qh);
        sh += hp[p] + hp[8 + p];
      }
      const float wj = j < k ? s_w[j] : 1.0f;
      acc = __builtin_fmaf(wj, bf16_to_f32(sc[m]) * qh + bf16_to_f32(bc[m]) * sh, acc);
    }
  }
  acc = wave_sum_dpp(acc);
  if (lane == 0) {
    if (a.residual) acc += bf16_to_f32(a.residual[c_row]);
    a.y[c_row] = f32_to_bf16(acc);
  }
}

bool decode_gemv_supported(int H, int I, int E, int k, int S, bool int4) {
  return int4 && H == DH && I == DI && E <= 256 && k + S <= kSlots;
}

hipError_t launch_decode_gemv(const DecodeArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_dec_a", k_dec_a, dim3(DWG), dim3(DT), 0, s, a);
  MOE_LAUNCH("k_dec_b", k_dec_b, dim3(DWG), dim3(DT), 0, s, a);
  MOE_LAUNCH("k_dec_c", k_dec_c, dim3(DWG), dim3(DT), 0, s, a);
  return hipSuccess;
}

}  // namespace moe
