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
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

// ---- router logits for many tokens: z[T,E] = x[T,H] W[E,H]^T + b --------------------------
// bf16 activations: MFMA in fp16 with the fp32 router weights split into two fp16 planes,
// hi = fp16(w) and lo = fp16((w - hi) * 2^11), so w = hi + lo * 2^-11 to 22 bits (the lo
// plane is scaled to stay clear of fp16 subnormals). x converts exactly to fp16 (inside the
// fp16 range), every product is exact in fp32, and the two planes accumulate separately in
// fp32 before z = acc_hi + 2^-11 acc_lo, so the logits carry fp32-class error.
//
// The planes are stored in MFMA B-operand order (router_frag_bytes), so that a wave loads its
// weight fragments straight from memory into registers, 1 KB per load instruction: only x
// goes through LDS, read by all four waves, and the LDS traffic per MFMA is a third of
// staging both operands there. Tile: 64 tokens x 128 experts x a quarter of the reduction
// axis per workgroup; wave w takes all 64 tokens x experts 32w .. 32w+31 (two 32x32
// accumulators per plane). The four quarters of the reduction land in four partial logit
// arrays that the top-k adds in a fixed order, so the sum is the same whatever runs first.
// Side jobs: the fp16 copy of x for the expert GEMMs (expert tile 0, chunks in kChunkOrder)
// and zeroing this token block's histogram row (the top-k kernel adds into it).
constexpr float kLoScale = 2048.0f;  // lo plane = fp16((w - hi) * 2^11)
constexpr int kRouterEPad = 128;     // experts per router tile; planes are zero-padded to it

MOE_DEV void split2(float w, uint16_t &hi, uint16_t &lo) {
  const _Float16 h = (_Float16)w;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, (_Float16)((w - (float)h) * kLoScale));
}

size_t router_frag_bytes(int E, int H) {
  const size_t ep = (size_t)(E + kRouterEPad - 1) / kRouterEPad * kRouterEPad;
  return 2 * ep * (size_t)H * 2;
}

// Router weights split into the two fp16 planes, in B-fragment order:
//   [E_pad / 32 column blocks][H / 16 K steps][plane hi, lo][64 lanes][8 halves]
// where lane l of (column block c, K step s) holds expert 32c + l % 32 at k = 16 s + 8 (l / 32)
// .. +7 (the v_mfma_f32_32x32x16_f16 B operand layout); experts past E are zero. Written once
// by moe_pack_weights, else on every call into the workspace. One thread per (c, s, lane).
__global__ __launch_bounds__(256) void k_router_split(const float *__restrict__ W, int E, int H,
                                                      uint16_t *__restrict__ planes) {
  const int ep = (E + kRouterEPad - 1) / kRouterEPad * kRouterEPad;
  const int ks = H / 16;
  const int n = ep / 32 * ks * 64;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int lane = i & 63, cs = i >> 6, st = cs % ks, c = cs / ks;
    const int e = 32 * c + (lane & 31), k = 16 * st + 8 * (lane >> 5);
    float v[8] = {};
    if (e < E) {
      const float4 a = *reinterpret_cast<const float4 *>(W + (size_t)e * H + k);
      const float4 b = *reinterpret_cast<const float4 *>(W + (size_t)e * H + k + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    uint16_t h[8], l[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) split2(v[q], h[q], l[q]);
    uint4 hv, lv;
    hv.x = h[0] | ((uint32_t)h[1] << 16); hv.y = h[2] | ((uint32_t)h[3] << 16);
    hv.z = h[4] | ((uint32_t)h[5] << 16); hv.w = h[6] | ((uint32_t)h[7] << 16);
    lv.x = l[0] | ((uint32_t)l[1] << 16); lv.y = l[2] | ((uint32_t)l[3] << 16);
    lv.z = l[4] | ((uint32_t)l[5] << 16); lv.w = l[6] | ((uint32_t)l[7] << 16);
    uint16_t *dst = planes + ((size_t)(c * ks + st) * 2) * 512 + 8 * lane;
    *reinterpret_cast<uint4 *>(dst) = hv;
    *reinterpret_cast<uint4 *>(dst + 512) = lv;
  }
}

// x tile in LDS: 64 rows x 64 fp16 of one K step, 16-byte chunk c of row r at chunk
// c ^ ((r >> 1) & 7), so the A-operand reads (16 rows of a 32-row block, one chunk) hit
// distinct banks.
MOE_DEV int router_a_off(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }

__global__ __launch_bounds__(256, 2) void k_router_mfma(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ planes,
                                                        const float *__restrict__ bias,
                                                        float *__restrict__ z,
                                                        uint16_t *__restrict__ x16,
                                                        int32_t *__restrict__ blk_cnt, int T,
                                                        int H, int E) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][64 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * kRouterEPad, kq = blockIdx.z;
  const int KQ = H / kRouterParts, kbase = kq * KQ, nsteps = KQ / 64, ks = H / 16;
  if (blockIdx.y == 0 && kq == 0)
    for (int e = tid; e < E; e += 256) blk_cnt[(size_t)blockIdx.x * E + e] = 0;
  // x staging: thread t loads chunks 2 (t % 4), +1 (8 elements each) of row t / 4
  const int lr = tid >> 2, lc = 2 * (tid & 3);
  const bool row_ok = t0 + lr < T;
  const uint16_t *xrow = x + (size_t)(row_ok ? t0 + lr : 0) * H + kbase + 8 * lc;
  // this wave's weight fragments: column block (e0 + 32 wave) / 32, 8 KB per K step
  const uint16_t *bsrc = planes + ((size_t)((e0 >> 5) + wave) * ks * 2) * 512 + 8 * lane;
  uint4 ra[2];
  uint4 bq[2][8];  // fragment sets of even and odd steps
  auto load_a = [&](int st) {
    const uint4 *p = reinterpret_cast<const uint4 *>(xrow + st * 64);
    ra[0] = row_ok ? p[0] : make_uint4(0, 0, 0, 0);
    ra[1] = row_ok ? p[1] : make_uint4(0, 0, 0, 0);
  };
  auto load_b = [&](int st, uint4 (&b)[8]) {
    const uint4 *p = reinterpret_cast<const uint4 *>(bsrc + (size_t)((kbase + st * 64) >> 4) * 1024);
#pragma unroll
    for (int q = 0; q < 8; ++q) b[q] = p[q * 64];  // (K step 4 st + q / 2, plane q % 2)
  };
  auto store_a = [&](int st) {
    uint16_t *as = As[st & 1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 u = ra[h];
      *reinterpret_cast<uint4 *>(as + router_a_off(lr, lc + h)) =
          make_uint4(bf16x2_to_f16x2(u.x), bf16x2_to_f16x2(u.y), bf16x2_to_f16x2(u.z),
                     bf16x2_to_f16x2(u.w));
      if (x16 && blockIdx.y == 0 && row_ok)
        *reinterpret_cast<uint4 *>(x16 + (size_t)(t0 + lr) * H + kbase + st * 64 + 8 * (lc + h)) =
            bf16x8_to_f16x8_chunk(u);
    }
  };
  f32x16_t acc_h[2] = {}, acc_l[2] = {};
  const int arow = lane & 31, ahalf = lane >> 5;
  auto compute = [&](int st, const uint4 (&b)[8]) {
    const uint16_t *as = As[st & 1];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f16x8_t bh = __builtin_bit_cast(f16x8_t, b[2 * kk]);
      const f16x8_t bl = __builtin_bit_cast(f16x8_t, b[2 * kk + 1]);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const f16x8_t av = *reinterpret_cast<const f16x8_t *>(
            as + router_a_off(32 * m + arow, 2 * kk + ahalf));
        acc_h[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bh, acc_h[m], 0, 0, 0);
        acc_l[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bl, acc_l[m], 0, 0, 0);
      }
    }
  };
  // steps in pairs: even steps use x stage 0 and fragment set 0, odd steps stage 1 and set 1;
  // the next step's x is stored while the current one computes (its stage was last read
  // before the previous barrier), and each set is reloaded right after its step's MFMAs.
  // (Fragments further ahead would need a third register set, which does not fit beside
  // the accumulators at two workgroups per CU.)
  load_a(0);
  load_b(0, bq[0]);
  store_a(0);
  if (nsteps > 1) {
    load_a(1);
    load_b(1, bq[1]);
  }
  __syncthreads();
  for (int st = 0; st < nsteps; st += 2) {
    compute(st, bq[0]);
    if (st + 1 < nsteps) store_a(st + 1);
    if (st + 2 < nsteps) {
      load_a(st + 2);
      load_b(st + 2, bq[0]);
    }
    __syncthreads();
    if (st + 1 >= nsteps) break;
    compute(st + 1, bq[1]);
    if (st + 2 < nsteps) store_a(st + 2);
    if (st + 3 < nsteps) {
      load_a(st + 3);
      load_b(st + 3, bq[1]);
    }
    __syncthreads();
  }
  // 32x32 accumulator layout: lane l holds column l % 32, register r row 8 (r / 4) + 4 (l / 32)
  // + r % 4 of the block. The bias is read once, outside the stores' branches (a load first
  // used inside them would make every store wait for all memory operations in flight).
  const int ee = e0 + 32 * wave + (lane & 31);
  float bv = 0.f;
  if (kq == 0 && bias) bv = bias[min(ee, E - 1)];
  asm volatile("" ::"v"(bv));
  float *zo = z + (size_t)kq * T * E;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = t0 + 32 * m + 8 * (r >> 2) + 4 * ahalf + (r & 3);
      const float v = __builtin_fmaf(acc_l[m][r], 1.0f / kLoScale, acc_h[m][r]) + bv;
      if (tt < T && ee < E) zo[(size_t)tt * E + ee] = v;
    }
}

// fp32 activations (fp32-weight layers): plain fp32 FMA on the vector ALUs.
__global__ __launch_bounds__(256) void k_router_f32(const float *__restrict__ x,
                                                    const float *__restrict__ W,
                                                    const float *__restrict__ bias,
                                                    float *__restrict__ z,
                                                    int32_t *__restrict__ blk_cnt, int T, int H,
                                                    int E) {
  __shared__ float xs[32][68];
  __shared__ float wsm[32][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  // 64 tokens x 64 experts over the whole reduction axis; zeroes this block's histogram slice
  if (tid < 64 && e0 + tid < E) blk_cnt[(size_t)blockIdx.x * E + e0 + tid] = 0;
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
      const float4 *p = reinterpret_cast<const float4 *>(x + (size_t)t * H + k0 + lk);
      const float4 a = p[0], b = p[1];
      xr[0] = a.x; xr[1] = a.y; xr[2] = a.z; xr[3] = a.w;
      xr[4] = b.x; xr[5] = b.y; xr[6] = b.z; xr[7] = b.w;
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
  // the biases are read once, outside the stores' branches (a load first used inside them
  // would make every store wait for memory)
  float bj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bj[j] = bias ? bias[min(e0 + tx * 4 + j, E - 1)] : 0.f;
  asm volatile("" ::"v"(bj[0]), "v"(bj[1]), "v"(bj[2]), "v"(bj[3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) z[(size_t)t * E + e] = acc[i][j] + bj[j];
    }
  }
}

// ---- top-k, one wave per token; per-block histogram by device atomics -----------------
// Workgroup = 4 waves = 4 tokens. blk_cnt[t / 64][e] was zeroed by the router kernel.
// kParts partial logit arrays of [T, E] each, contiguous, added in index order.
template <int kParts>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ z, int T, int E, int k,
                                              int32_t *__restrict__ ids,
                                              float *__restrict__ w,
                                              int32_t *__restrict__ blk_cnt) {
  __shared__ __attribute__((aligned(16))) uint64_t s_topk[4][kTopkScratch];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  // all loads leave before the first use (experts past E read the last one and are masked)
  float p[kParts][4];
#pragma unroll
  for (int q = 0; q < kParts; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      p[q][c] = z[(size_t)q * T * E + (size_t)t * E + min(lane + kWave * c, E - 1)];
  float v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[c] = p[0][c];
#pragma unroll
    for (int q = 1; q < kParts; ++q) v[c] += p[q][c];
    if (lane + kWave * c >= E) v[c] = -INFINITY;
  }
  int id, pos;
  float weight;
  wave_topk(v, E, k, s_topk[wave], id, pos, weight);
  if (lane < k) {
    ids[(size_t)t * k + pos] = id;
    w[(size_t)t * k + pos] = weight;
    atomicAdd(&blk_cnt[(size_t)(t / kRouteBlock) * E + id], 1);
  }
}

// Inclusive block-wide scan over 256 threads (LDS, Hillis-Steele).
// Inclusive scan over the 256 threads of the workgroup: shuffle scan inside each wave,
// then the totals of the waves before it (one LDS exchange, two barriers).
template <typename V>
MOE_DEV V block_scan_incl(V v, V *wtot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const V o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  V before = 0;
  for (int w = 0; w < wave; ++w) before += wtot[w];
  __syncthreads();  // wtot may be reused by the next scan
  return v + before;
}

// ---- counts, offsets and the tile map from the per-expert totals --------------------------
// Called by all 256 threads of a workgroup; thread e < E passes run = the assignments to expert
// e (others 0). Returns the exclusive prefix of run over the experts (the group offset of e).
// With `write` set the workgroup also stores the offsets (E+2 entries: routed experts, then the
// shared expert's slots [kT, kT+T)), the caller's counts and offsets, and the tile map.
MOE_DEV int group_tables(int run, bool write, int E, int T, int S, int32_t *__restrict__ offsets,
                         int32_t *__restrict__ counts_user, int32_t *__restrict__ offsets_user,
                         int2 *__restrict__ tiles, int32_t *__restrict__ n_tiles, int tsh_fixed,
                         int fill) {
  const int e = threadIdx.x;
  // one scan gives the offsets (low word) and the number of 32-row blocks the experts'
  // rows fill (high word)
  __shared__ uint64_t sc64[4];
  const uint64_t rb = (uint64_t)run | ((uint64_t)((run + 31) >> 5) << 32);
  const uint64_t rincl = block_scan_incl(rb, sc64);
  const int off = (int)((rincl - rb) & 0xFFFFFFFFu);
  __shared__ uint64_t rtot[1];
  if (e == 255) rtot[0] = rincl;
  __syncthreads();
  const int nassign = (int)(rtot[0] & 0xFFFFFFFFu);
  // Tile height of this call, from the load ("Match tile size to expert load"): while the
  // rows fill at least 4 * fill blocks (fill = 32-row blocks per resident gate/up
  // workgroup slot of one N tile), 128-row tiles; with fewer, a 128-row tile would outlast
  // the rest of the grid, so 64 rows (at least 2 * fill blocks) or 32. Callers may fix it.
  int tsh = tsh_fixed;
  if (tsh <= 0) {
    const int nblk = (int)(rtot[0] >> 32) + (S ? (T + 31) >> 5 : 0);
    tsh = nblk >= 4 * fill ? 7 : nblk >= 2 * fill ? 6 : 5;
  }
  // Tile map in descending order of work (the GEMM workgroups start in index order, so the
  // long tiles go first and the short ones fill the end): every full tile of 2^tsh rows
  // (routed experts in order, then the shared expert), then the partial tiles by their
  // number of 32-row blocks, 4 down to 1: each expert's last tile is only as high as its
  // remaining rows need. With 128-row tiles chosen from the load, a remainder of at most
  // 32 rows joins the group's last full tile instead (one tile of 129..160 rows, five
  // blocks, rather than a one-block tile that would pay the whole weight tile's loads for a
  // quarter of the work). One 64-bit scan places them all: bits [0, 22) count full tiles,
  // 9-bit fields at 22 + 9q count partial tiles of 4 - q blocks. A tile entry is
  // (group | rows << 16, first row).
  const int trows = 1 << tsh;
  const bool merge = tsh_fixed <= 0 && tsh == 7;
  const int nfull = run >> tsh;
  int rem = run & (trows - 1), last = trows;
  if (merge && nfull > 0 && rem > 0 && rem <= 32) {
    last = trows + rem;
    rem = 0;
  }
  const int mb = (rem + 31) >> 5;
  const uint64_t packed = (uint64_t)nfull | (mb ? (1ull << (22 + 9 * (4 - mb))) : 0ull);
  const uint64_t pincl = block_scan_incl(packed, sc64);
  if (!write) return off;
  const uint64_t pexcl = pincl - packed;
  __shared__ uint64_t ptot[1];
  if (e == 255) ptot[0] = pincl;
  __syncthreads();
  const uint64_t tot = ptot[0];
  const int nfull_tot = (int)(tot & 0x3FFFFF);
  const int sh_full = S ? T >> tsh : 0;
  int sh_rem = S ? (T & (trows - 1)) : 0, sh_last = trows;
  if (merge && sh_full > 0 && sh_rem > 0 && sh_rem <= 32) {
    sh_last = trows + sh_rem;
    sh_rem = 0;
  }
  int bstart[4];
  bstart[0] = nfull_tot + sh_full;
#pragma unroll
  for (int q = 1; q < 4; ++q) bstart[q] = bstart[q - 1] + (int)((tot >> (22 + 9 * (q - 1))) & 0x1FF);
  const int npart = bstart[3] + (int)((tot >> (22 + 27)) & 0x1FF);
  if (e < E) {
    offsets[e] = off;
    if (counts_user) counts_user[e] = run;
    if (offsets_user) offsets_user[e] = off;
    const int f0 = (int)(pexcl & 0x3FFFFF);
    for (int i = 0; i < nfull; ++i)
      tiles[f0 + i] = make_int2(e | (i + 1 < nfull ? trows : last) << 16, i * trows);
    if (mb) {
      const int q = 4 - mb;
      tiles[bstart[q] + (int)((pexcl >> (22 + 9 * q)) & 0x1FF)] =
          make_int2(e | rem << 16, nfull * trows);
    }
  }
  for (int i = e; i < sh_full; i += 256)
    tiles[nfull_tot + i] = make_int2(E | (i + 1 < sh_full ? trows : sh_last) << 16, i * trows);
  if (e == 0) {
    if (sh_rem) tiles[npart] = make_int2(E | sh_rem << 16, sh_full * trows);
    offsets[E] = nassign;
    offsets[E + 1] = nassign + (S ? T : 0);
    if (offsets_user) offsets_user[E] = nassign;
    *n_tiles = npart + (sh_rem ? 1 : 0);
  }
  return off;
}

// Per-chunk expert counts for long calls: workgroup c adds the block rows of chunk c
// (kChunkBlocks routing blocks), thread e its expert's column, in block order.
__global__ __launch_bounds__(256) void k_chunk_sum(const int32_t *__restrict__ blk_cnt, int NB,
                                                   int E, int32_t *__restrict__ chunk_cnt) {
  const int c = blockIdx.x, e = threadIdx.x;
  if (e >= E) return;
  const int b0 = c * kChunkBlocks, b1 = min(NB, b0 + kChunkBlocks);
  int v[kChunkBlocks];
#pragma unroll
  for (int i = 0; i < kChunkBlocks; ++i) v[i] = b0 + i < b1 ? blk_cnt[(size_t)(b0 + i) * E + e] : 0;
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kChunkBlocks; ++i) sum += v[i];
  chunk_cnt[(size_t)c * E + e] = sum;
}

// Scan and scatter in one kernel, one workgroup per routing block of 64 tokens: thread e sums
// the block counts of expert e over all blocks (its total) and over the blocks before this one
// (its base), every workgroup forms the same offsets from the totals (same inputs, same
// order), workgroup 0 also writes the tables, and the block's assignments are placed as in
// k_scatter. The histogram is only read, so the workgroups need no ordering between them.
template <bool kChunked>
__global__ __launch_bounds__(256) void k_group(const int32_t *__restrict__ blk_cnt,
                                               const int32_t *__restrict__ chunk_cnt,
                                               const int32_t *__restrict__ ids,
                                               const float *__restrict__ w, int NB, int E, int T,
                                               int k, int S, int32_t *__restrict__ offsets,
                                               int32_t *__restrict__ counts_user,
                                               int32_t *__restrict__ offsets_user,
                                               int2 *__restrict__ tiles,
                                               int32_t *__restrict__ n_tiles, int tsh_fixed,
                                               int fill, int32_t *__restrict__ sorted_tok,
                                               int32_t *__restrict__ slot_of,
                                               float *__restrict__ slot_w,
                                               int32_t *__restrict__ sync, int n_sync) {
  __shared__ unsigned long long mask[kMaxExperts];
  __shared__ int start[kMaxExperts];
  const int b = blockIdx.x, t0 = b * kRouteBlock, tid = threadIdx.x;
  // the fused GEMM launch's queue words start at zero
  for (int i = b * 256 + tid; i < n_sync; i += NB * 256) sync[i] = 0;
  // thread e: its expert's total over all blocks (run) and over the blocks before this one
  // (base). For long calls k_chunk_sum has added the block rows per chunk of kChunkBlocks
  // blocks: the totals then come from the chunk rows, and the base from the chunks before
  // this block's chunk plus at most kChunkBlocks - 1 block rows, so every workgroup reads
  // about T / 4096 + 64 rows instead of all T / 64. Integer sums: the same values either
  // way.
  int run = 0, base = 0;
  if (tid < E && !kChunked) {
    for (int b0 = 0; b0 < NB; b0 += 32) {
      int c[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) c[i] = b0 + i < NB ? blk_cnt[(size_t)(b0 + i) * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        base += b0 + i < b ? c[i] : 0;
        run += c[i];
      }
    }
  } else if (kChunked && tid < E) {
    const int NC = (NB + kChunkBlocks - 1) / kChunkBlocks, cb = b / kChunkBlocks;
    for (int c0 = 0; c0 < NC; c0 += 32) {
      int c[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) c[i] = c0 + i < NC ? chunk_cnt[(size_t)(c0 + i) * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        base += c0 + i < cb ? c[i] : 0;
        run += c[i];
      }
    }
    for (int b0 = cb * kChunkBlocks; b0 < b; b0 += 32) {  // this chunk's blocks before b
      int c[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) c[i] = b0 + i < b ? blk_cnt[(size_t)(b0 + i) * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) base += c[i];
    }
  }
  const int off = group_tables(run, b == 0, E, T, S, offsets, counts_user, offsets_user, tiles,
                               n_tiles, tsh_fixed, fill);
  start[tid] = off + base;
  mask[tid] = 0ull;
  __syncthreads();
  const int nt = min(kRouteBlock, T - t0), na = nt * k;
  for (int i = tid; i < na; i += 256) {
    const int e = ids[(size_t)t0 * k + i];
    atomicOr(&mask[e], 1ull << (i / k));
  }
  __syncthreads();
  for (int i = tid; i < na; i += 256) {
    const int tt = i / k, e = ids[(size_t)t0 * k + i];
    const unsigned long long before = tt ? (mask[e] & (~0ull >> (64 - tt))) : 0ull;
    const int slot = start[e] + __popcll(before);
    sorted_tok[slot] = t0 + tt;
    slot_of[(size_t)t0 * k + i] = slot;
    if (slot_w) slot_w[slot] = w[(size_t)t0 * k + i];
  }
}

// ---- stable scatter: slot of every assignment ---------------------------------------
// One workgroup per routing block of 64 tokens. mask[e] has bit tt set when token t0+tt
// chose expert e, so the rank of (t, j) inside its expert's run of this block is the
// number of earlier tokens in the mask: slot = offsets[e] + base[b][e] + rank.
__global__ __launch_bounds__(256) void k_scatter(const int32_t *__restrict__ ids, int T, int E,
                                                 int k, const int32_t *__restrict__ offsets,
                                                 const int32_t *__restrict__ blk_base,
                                                 const float *__restrict__ w,
                                                 int32_t *__restrict__ sorted_tok,
                                                 int32_t *__restrict__ slot_of,
                                                 float *__restrict__ slot_w) {
  __shared__ unsigned long long mask[kMaxExperts];
  const int b = blockIdx.x, t0 = b * kRouteBlock, tid = threadIdx.x;
  const int nt = min(kRouteBlock, T - t0), na = nt * k;
  mask[tid] = 0ull;
  __syncthreads();
  for (int i = tid; i < na; i += 256) {
    const int e = ids[(size_t)t0 * k + i];
    atomicOr(&mask[e], 1ull << (i / k));
  }
  __syncthreads();
  for (int i = tid; i < na; i += 256) {
    const int tt = i / k, e = ids[(size_t)t0 * k + i];
    const unsigned long long before = tt ? (mask[e] & (~0ull >> (64 - tt))) : 0ull;
    const int slot = offsets[e] + blk_base[(size_t)b * E + e] + __popcll(before);
    sorted_tok[slot] = t0 + tt;
    slot_of[(size_t)t0 * k + i] = slot;
    if (slot_w) slot_w[slot] = w[(size_t)t0 * k + i];
  }
}

// ---- launchers ------------------------------------------------------------------------------
hipError_t launch_router_split(const float *W, int E, int H, uint16_t *planes, hipStream_t s) {
  const int n = (E + kRouterEPad - 1) / kRouterEPad * kRouterEPad / 32 * (H / 16) * 64;
  MOE_LAUNCH("k_router_split", k_router_split, dim3((unsigned)std::min((n + 255) / 256, 2048)),
             dim3(256), 0, s, W, E, H, planes);
  return hipSuccess;
}

hipError_t launch_route_topk(const RouteArgs &a, hipStream_t s) {
  const int NB = (int)((a.T + kRouteBlock - 1) / kRouteBlock);
  if (a.bf16) {
    if (!a.planes_ready) {
      const hipError_t e = launch_router_split(a.router_w, a.E, a.H, a.router_planes, s);
      if (e != hipSuccess) return e;
    }
    MOE_LAUNCH("k_router_mfma", k_router_mfma,
               dim3((unsigned)NB, (unsigned)((a.E + kRouterEPad - 1) / kRouterEPad), kRouterParts),
               dim3(256), 0, s, static_cast<const uint16_t *>(a.x), a.router_planes, a.router_b,
               a.logits, a.x16, a.blk, (int)a.T, a.H, a.E);
    MOE_LAUNCH("k_topk", k_topk<kRouterParts>, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s,
               a.logits, (int)a.T, a.E, a.k, a.ids, a.w, a.blk);
  } else {
    MOE_LAUNCH("k_router_f32", k_router_f32, dim3((unsigned)NB, (unsigned)((a.E + 63) / 64)),
               dim3(256), 0, s, static_cast<const float *>(a.x), a.router_w, a.router_b,
               a.logits, a.blk, (int)a.T, a.H, a.E);
    MOE_LAUNCH("k_topk", k_topk<1>, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s, a.logits,
               (int)a.T, a.E, a.k, a.ids, a.w, a.blk);
  }
  return hipSuccess;
}

hipError_t launch_route_scatter(const RouteArgs &a, hipStream_t s) {
  const int NB = (int)((a.T + kRouteBlock - 1) / kRouteBlock);
  MOE_LAUNCH("k_scatter", k_scatter, dim3(NB), dim3(256), 0, s, a.ids, (int)a.T, a.E, a.k,
             a.offsets, a.blk, a.w, a.sorted_tok, a.slot_of, a.slot_w);
  return hipSuccess;
}

hipError_t launch_route_prefill(const RouteArgs &a, hipStream_t s) {
  const hipError_t e = launch_route_topk(a, s);
  if (e != hipSuccess) return e;
  const int NB = (int)((a.T + kRouteBlock - 1) / kRouteBlock);
  if (a.chunk) {
    MOE_LAUNCH("k_chunk_sum", k_chunk_sum, dim3((unsigned)((NB + kChunkBlocks - 1) / kChunkBlocks)),
               dim3(256), 0, s, a.blk, NB, a.E, a.chunk);
    MOE_LAUNCH("k_group", k_group<true>, dim3(NB), dim3(256), 0, s, a.blk, a.chunk, a.ids, a.w,
               NB, a.E, (int)a.T, a.k, a.S, a.offsets, a.counts_user, a.offsets_user, a.tiles,
               a.n_tiles, a.tile_shift, gemm_fill(a.I), a.sorted_tok, a.slot_of, a.slot_w, a.sync,
               a.n_sync);
  } else {
    MOE_LAUNCH("k_group", k_group<false>, dim3(NB), dim3(256), 0, s, a.blk, a.chunk, a.ids, a.w,
               NB, a.E, (int)a.T, a.k, a.S, a.offsets, a.counts_user, a.offsets_user, a.tiles,
               a.n_tiles, a.tile_shift, gemm_fill(a.I), a.sorted_tok, a.slot_of, a.slot_w, a.sync,
               a.n_sync);
  }
  return hipSuccess;
}

}  // namespace moe
