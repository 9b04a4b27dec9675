// route.hip -- router logits, top-k with renormalised softmax, and grouping of the
// token-expert assignments by expert, all on the GPU.
//
// "Optimizing On-Device Inference for Apple Silicon":
//   section "Qwen creates three distinct workload shapes" -- the router scores every
//   expert and keeps eight per token;
//   section "Keep expert routing on the GPU" -- a histogram of assignments per expert,
//   a prefix scan into start offsets, a scatter into expert groups and a map of the
//   fixed-size blocks the grouped GEMM processes, with no CPU round trip.
//
// The scatter here is a stable counting sort (tokens ascending within an expert), so
// the grouping is a pure function of the routing: no atomics decide any position.
#include "common.h"
#include "kernels.h"

namespace moe {

// ---- router logits for many tokens: z[T,E] = x[T,H] W[E,H]^T + b ------------------------
// 64 tokens x 64 experts per workgroup, fp32 FMA on the vector ALUs, K staged in LDS
// in chunks of 32. Each thread owns a 4x4 block of outputs.
template <bool kBf16>
__global__ __launch_bounds__(256) void k_router_logits(const void *__restrict__ xv,
                                                       const float *__restrict__ W,
                                                       const float *__restrict__ bias,
                                                       float *__restrict__ z,
                                                       uint16_t *__restrict__ x16, int T, int H,
                                                       int E) {
  __shared__ float xs[32][68];
  __shared__ float wsm[32][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int lr = tid >> 2, lk = (tid & 3) * 8;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < H; k0 += 32) {
    float xr[8], wr[8];
    const int t = t0 + lr, e = e0 + lr;
    if (t < T) {
      if (kBf16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(
            static_cast<const uint16_t *>(xv) + (size_t)t * H + k0 + lk);
        xr[0] = bf16lo(u.x); xr[1] = bf16hi(u.x); xr[2] = bf16lo(u.y); xr[3] = bf16hi(u.y);
        xr[4] = bf16lo(u.z); xr[5] = bf16hi(u.z); xr[6] = bf16lo(u.w); xr[7] = bf16hi(u.w);
        if (x16 && blockIdx.y == 0) {
          // fp16 copy of x for the fp16 MFMA GEMMs (exact inside the fp16 range)
          uint4 h;
          h.x = bf16x2_to_f16x2(u.x);
          h.y = bf16x2_to_f16x2(u.y);
          h.z = bf16x2_to_f16x2(u.z);
          h.w = bf16x2_to_f16x2(u.w);
          *reinterpret_cast<uint4 *>(x16 + (size_t)t * H + k0 + lk) = h;
        }
      } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(xv) +
                                                           (size_t)t * H + k0 + lk);
        const float4 a = p[0], b = p[1];
        xr[0] = a.x; xr[1] = a.y; xr[2] = a.z; xr[3] = a.w;
        xr[4] = b.x; xr[5] = b.y; xr[6] = b.z; xr[7] = b.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xr[i] = 0.f;
    }
    if (e < E) {
      const float4 *p = reinterpret_cast<const float4 *>(W + (size_t)e * H + k0 + lk);
      const float4 a = p[0], b = p[1];
      wr[0] = a.x; wr[1] = a.y; wr[2] = a.z; wr[3] = a.w;
      wr[4] = b.x; wr[5] = b.y; wr[6] = b.z; wr[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) wr[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xs[lk + i][lr] = xr[i];
      wsm[lk + i][lr] = wr[i];
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      const float4 a = *reinterpret_cast<const float4 *>(&xs[kk][ty * 4]);
      const float4 b = *reinterpret_cast<const float4 *>(&wsm[kk][tx * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) z[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
    }
  }
}

// ---- top-k and per-block histogram for T tokens -----------------------------------------
// One workgroup per routing block of 64 tokens; each wave handles 16 tokens in order.
__global__ __launch_bounds__(256) void k_topk_hist(const float *__restrict__ z, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w,
                                                   int32_t *__restrict__ blk_cnt) {
  __shared__ int hist[kMaxExperts];
  __shared__ __attribute__((aligned(16))) uint64_t s_topk[4][kTopkScratch];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  hist[tid] = 0;
  __syncthreads();
  const int tbase = blockIdx.x * kRouteBlock + wave * 16;
  for (int tt = 0; tt < 16; ++tt) {
    const int t = tbase + tt;
    if (t >= T) break;
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + kWave * c;
      v[c] = e < E ? z[(size_t)t * E + e] : -INFINITY;
    }
    int sel[kMaxTopK];
    float sw[kMaxTopK];
    wave_topk(v, E, k, s_topk[wave], sel, sw);
    int id = 0;
    float weight = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j == lane) {
        id = sel[j];
        weight = sw[j];
      }
    if (lane < k) {
      ids[(size_t)t * k + lane] = id;
      w[(size_t)t * k + lane] = weight;
      atomicAdd(&hist[id], 1);
    }
  }
  __syncthreads();
  if (tid < E) blk_cnt[(size_t)blockIdx.x * E + tid] = hist[tid];
}

// Inclusive block-wide scan over 256 threads (LDS, Hillis-Steele).
MOE_DEV int block_scan_incl(int v, int *sc) {
  const int tid = threadIdx.x;
  sc[tid] = v;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int o = tid >= d ? sc[tid - d] : 0;
    __syncthreads();
    sc[tid] += o;
    __syncthreads();
  }
  const int r = sc[tid];
  __syncthreads();
  return r;
}

// ---- counts, offsets, per-block bases and the tile map (one workgroup) -------------------
// blk_cnt[b][e] becomes the number of assignments to e in blocks before b. offsets has
// E+2 entries: routed experts, then the shared expert's slots [kT, kT+T).
__global__ __launch_bounds__(256) void k_scan(int32_t *__restrict__ blk_cnt, int NB, int E,
                                              int T, int k, int S,
                                              int32_t *__restrict__ offsets,
                                              int32_t *__restrict__ counts_user,
                                              int32_t *__restrict__ offsets_user,
                                              int2 *__restrict__ tiles,
                                              int32_t *__restrict__ n_tiles) {
  __shared__ int sc[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int b = 0; b < NB; ++b) {
      const int c = blk_cnt[(size_t)b * E + e];
      blk_cnt[(size_t)b * E + e] = run;
      run += c;
    }
  }
  const int incl = block_scan_incl(run, sc);
  const int off = incl - run;
  const int ntile = (run + kTileM - 1) / kTileM;
  const int tincl = block_scan_incl(ntile, sc);
  const int tstart = tincl - ntile;
  __shared__ int totals[2];
  if (e == 255) {
    totals[0] = incl;
    totals[1] = tincl;
  }
  __syncthreads();
  const int nassign = totals[0], nt_routed = totals[1];
  if (e < E) {
    offsets[e] = off;
    if (counts_user) counts_user[e] = run;
    if (offsets_user) offsets_user[e] = off;
    for (int i = 0; i < ntile; ++i) tiles[tstart + i] = make_int2(e, i * kTileM);
  }
  const int nt_shared = S ? (T + kTileM - 1) / kTileM : 0;
  for (int i = e; i < nt_shared; i += 256) tiles[nt_routed + i] = make_int2(E, i * kTileM);
  if (e == 0) {
    offsets[E] = nassign;
    offsets[E + 1] = nassign + (S ? T : 0);
    if (offsets_user) offsets_user[E] = nassign;
    *n_tiles = nt_routed + nt_shared;
  }
}

// ---- stable scatter: slot of every assignment --------------------------------------------
__global__ __launch_bounds__(256) void k_scatter(const int32_t *__restrict__ ids, int T, int E,
                                                 int k, const int32_t *__restrict__ offsets,
                                                 const int32_t *__restrict__ blk_base,
                                                 const float *__restrict__ w,
                                                 int32_t *__restrict__ sorted_tok,
                                                 int32_t *__restrict__ slot_of,
                                                 float *__restrict__ slot_w) {
  __shared__ int sid[kRouteBlock * kMaxTopK];
  const int b = blockIdx.x, t0 = b * kRouteBlock;
  const int nt = min(kRouteBlock, T - t0);
  for (int i = threadIdx.x; i < nt * k; i += 256) sid[i] = ids[(size_t)t0 * k + i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int slot = offsets[e] + blk_base[(size_t)b * E + e];
    for (int tt = 0; tt < nt; ++tt) {
      for (int j = 0; j < k; ++j) {
        if (sid[tt * k + j] == e) {
          sorted_tok[slot] = t0 + tt;
          slot_of[(size_t)(t0 + tt) * k + j] = slot;
          if (slot_w) slot_w[slot] = w[(size_t)(t0 + tt) * k + j];
          ++slot;
        }
      }
    }
  }
}

// ---- launchers ------------------------------------------------------------------------------
hipError_t launch_route_prefill(const RouteArgs &a, hipStream_t s) {
  const int NB = (int)((a.T + kRouteBlock - 1) / kRouteBlock);
  dim3 g1((unsigned)((a.T + 63) / 64), (unsigned)((a.E + 63) / 64));
  if (a.bf16)
    MOE_LAUNCH("k_router_logits", (k_router_logits<true>), g1, dim3(256), 0, s, a.x,
               a.router_w, a.router_b, a.logits, a.x16, (int)a.T, a.H, a.E);
  else
    MOE_LAUNCH("k_router_logits", (k_router_logits<false>), g1, dim3(256), 0, s, a.x,
               a.router_w, a.router_b, a.logits, nullptr, (int)a.T, a.H, a.E);
  MOE_LAUNCH("k_topk_hist", k_topk_hist, dim3(NB), dim3(256), 0, s, a.logits, (int)a.T, a.E,
             a.k, a.ids, a.w, a.blk);
  MOE_LAUNCH("k_scan", k_scan, dim3(1), dim3(256), 0, s, a.blk, NB, a.E, (int)a.T, a.k, a.S,
             a.offsets, a.counts_user, a.offsets_user, a.tiles, a.n_tiles);
  MOE_LAUNCH("k_scatter", k_scatter, dim3(NB), dim3(256), 0, s, a.ids, (int)a.T, a.E, a.k,
             a.offsets, a.blk, a.w, a.sorted_tok, a.slot_of, a.slot_w);
  return hipSuccess;
}

}  // namespace moe
