// decode_gemv.hip -- batch-1 MoE layer (hidden 2048, intermediate 512, int4 g64) in three
// lean kernels on the vector ALUs, reading the tiled weight layout of moe_pack_weights.
//
// "Optimizing On-Device Inference for Apple Silicon":
//   section "Decode: minimize the bytes moved per token" -- only the router, the k
//   selected experts and the shared expert are read, each byte once;
//   section "Optimize the one-row weight path" -- row-parallel GEMVs whose lanes read
//   adjacent 16-byte pieces: in the tiled layout one load instruction of a wave is one
//   contiguous 1 KB block (32 rows x 32 code bytes of one K step);
//   section "Overlap independent GPU work" -- the shared expert does not depend on the
//   routing, so its gate/up projection runs next to the top-k;
//   section "Reduce intermediate and state traffic" -- gate/up are fused with SwiGLU and
//   the output projection with the routing weights and the shared-expert result.
//
// The kernel boundaries are the two device-wide exchanges the layer needs (all router
// logits before the top-k, all of h before the output projection). Inside a HIP graph a
// boundary costs about 1.4 us on MI355X, less than a grid barrier built on device-scope
// atomics across 256 workgroups (2.4-3.7 us), so no kernel spins.
//
//   A  256 workgroups: workgroup w computes router logit z[w].
//   B  256 workgroups run the top-k on z (same data, same code, same answer), then
//      compute 16 gate + 16 up rows of one selected expert: workgroup (slot j, block b,
//      half f) -> rows 32b + 16f .. +16, slot j being the j-th largest logit. Workgroup 0
//      stores the selected ids and logits for C. 32 more workgroups compute the shared
//      expert's gate/up the same way; they need no routing, so they skip the top-k and
//      overlap it.
//   C  512 workgroups of 4 output rows each: all k+1 experts' W2 rows times h (staged
//      in LDS), scaled by the routing weights (the softmax over the selected logits, formed
//      while the W2 rows are in flight), plus the residual.
//
// Dot products: a nibble pair OR-ed into 0x6400 is the fp16 pair (1024 + q_lo, 1024 + q_hi)
// of elements (8m + p, 8m + p + 4) of a 32-bit code word m; the activations sit in LDS as
// fp16 pairs in the same order, so v_dot2_f32_f16 multiplies exactly and accumulates in
// fp32, and per quantisation group sum (s q + b) x = s * dot + (b - 1024 s) * sum(x), all
// in fp32. Activations must lie inside the fp16 range.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int DH = 2048, DI = 512, DWG = 256, DT = 512;
constexpr int kSlots = kMaxTopK + 1;
constexpr int kNB13 = 2 * DI / 64;  // 64-row blocks of W13 (32 gate + 32 up rows)
constexpr int kNS13 = DH / 64;      // K steps of W13
constexpr int kNB2 = DH / 64;       // 64-row blocks of W2
constexpr int kNS2 = DI / 64;       // K steps of W2
constexpr int kSharedWG = 2 * kNB13; // extra workgroups of B: shared-expert half blocks
constexpr int kDownWG = kNB2 * 16;  // C: 4 output rows per workgroup
static_assert(kNB2 % 8 == 0, "the down kernel spreads its 64-row blocks evenly over 8 XCDs");

// Down-projection workgroup w owns output rows 64b + 4t .. +4. The 16 workgroups of one
// 64-row block read 128-byte pieces of the same 2 KB code blocks and 64-byte pieces of the
// same scale blocks; workgroup ids are dealt round-robin over the 8 XCDs, so the ids are
// mapped to put all 16 on one XCD: every line is then fetched into one L2 once, instead of
// into several L2s by halves.
MOE_DEV void down_rows_of(int w, int &b, int &t) {
  const int j = w >> 3;
  b = (kNB2 / 8) * (w & 7) + (j >> 4);
  t = j & 15;
}
}  // namespace

// n fp32 / bf16 activations -> fp16 pairs (v[8c + p], v[8c + p + 4]) for chunk c, p < 4, in
// LDS, and the sum of each 32-element segment (of the fp16 values) in seg[n / 32]. Called
// by all DT threads (n a multiple of 32).
template <bool kBf16In>
MOE_DEV void stage_f16_pairs(const void *src, int n, f16x2_t *pairs, float *seg) {
  const int nchunks = n / 8;
  for (int base = 0; base < nchunks; base += DT) {
    const int ch = base + threadIdx.x;  // 8 elements
    const bool live = ch < nchunks;
    float v[8] = {};
    if (live) {
      if (kBf16In) {
        const uint4 u = reinterpret_cast<const uint4 *>(src)[ch];
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16lo(wd[i]);
          v[2 * i + 1] = bf16hi(wd[i]);
        }
      } else {
        const float4 a = reinterpret_cast<const float4 *>(src)[2 * ch];
        const float4 b = reinterpret_cast<const float4 *>(src)[2 * ch + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
    }
    float sum = 0.f;
    f16x2_t pr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      pr[p] = f16x2_t{(_Float16)v[p], (_Float16)v[p + 4]};
      sum += (float)pr[p][0] + (float)pr[p][1];
    }
    if (live) *reinterpret_cast<uint4 *>(pairs + 4 * ch) = __builtin_bit_cast(uint4, pr);
    // 4 chunks per segment: lanes 4s .. 4s+3 (DT is a multiple of 4)
    sum = xor_sum<1>(sum);
    sum = xor_sum<2>(sum);
    if ((ch & 3) == 0 && live) seg[ch >> 2] = sum;
  }
}

// The bf16 layer input as fp16 pairs in LDS plus its 32-element segment sums (of the fp16
// values): thread t < DH / 8 takes chunk t. With a.norm the input is the normalised row that
// k_dec_a wrote (a.xn), else x itself.
MOE_DEV void stage_x(const DecodeArgs &a, f16x2_t *pairs, float *seg) {
  const int tid = threadIdx.x;
  const bool live = tid < DH / 8;
  const uint16_t *src = a.norm ? a.xn : a.x;
  float v[8] = {};
  if (live) {
    const uint4 u = reinterpret_cast<const uint4 *>(src)[tid];
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16lo(wd[i]);
      v[2 * i + 1] = bf16hi(wd[i]);
    }
  }
  float sum = 0.f;
  f16x2_t pr[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    pr[p] = f16x2_t{(_Float16)v[p], (_Float16)v[p + 4]};
    sum += (float)pr[p][0] + (float)pr[p][1];
  }
  if (live) *reinterpret_cast<uint4 *>(pairs + 4 * tid) = __builtin_bit_cast(uint4, pr);
  sum = xor_sum<1>(sum);
  sum = xor_sum<2>(sum);
  if ((tid & 3) == 0 && live) seg[tid >> 2] = sum;
}

// Raw dot of one lane's 16 code bytes (32 elements = chunks c0 .. c0+3) with the staged
// fp16 pairs: sum over the elements of (1024 + q) * x.
MOE_DEV float dot_codes(const uint4 c, const f16x2_t *pairs, int c0) {
  constexpr uint32_t kMask = 0x000F000Fu, kMagic = 0x64006400u;
  const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint4 xp = *reinterpret_cast<const uint4 *>(pairs + 4 * (c0 + m));
    const uint32_t xs[4] = {xp.x, xp.y, xp.z, xp.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t t = and_or(wd[m] >> (4 * p), kMask, kMagic);
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, t),
                                   __builtin_bit_cast(f16x2_t, xs[p]), acc, false);
    }
  }
  return acc;
}

// (s q + b) . x of one group-step segment from the raw dot, scale/bias as bf16 bits
MOE_DEV float group_dot(float raw, uint32_t sb, float xsum) {
  const float sc = bf16lo(sb), bi = bf16hi(sb);
  return __builtin_fmaf(sc, raw, (bi - 1024.0f * sc) * xsum);
}

MOE_DEV uint32_t word_of(const uint4 v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Top-k of the E <= 256 router logits using all 8 waves of the workgroup (latency: the
// chain of dependent instructions is what costs time for a single wave). Keys are 64-bit:
// float key high, ~id low, so one unsigned compare orders by (logit desc, id asc).
//   1. wave v ranks elements [32v, 32v+32) among themselves (two lanes per element, 16
//      comparisons each); its k best go to cand[8v ..]. The wave loaded these logits
//      itself, so it needs no workgroup barrier, only the in-order LDS of one wave.
//   2. after one barrier the 64 candidates are ranked among each other (lane: candidate
//      8v + l%8 against comparands 8(l/8) .. 8(l/8)+7, partial ranks summed over the 8
//      lane groups); the winners land in K[0 .. k-1] in rank order, K[0] the largest.
// Must be called by all DT threads; thread t passes the logit of element 32 (t / 64) +
// t % 32 (loaded by the caller, so that the load can leave early). Needs E >= k.
MOE_DEV void block_topk(float zv, int E, int k, uint64_t *K, uint64_t *cand) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = 32 * wave + (lane & 31), half = lane >> 5;
  {
    const float g = (e >= E || zv != zv) ? -INFINITY : zv;
    const uint64_t mine =
        e < E ? ((uint64_t)float_key(g) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
    if (half == 0) K[e] = mine;
    if (lane < 8) cand[8 * wave + lane] = 0ull;
    wave_lds_sync();
    const uint64_t *base = K + 32 * wave + 16 * half;
    int r = 0;
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
      const ulonglong2 p = *reinterpret_cast<const ulonglong2 *>(base + q);
      r += (p.x > mine) + (p.y > mine);
    }
    r = xor_sum<32>(r);
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
    r = xor_sum<8>(r);
    r = xor_sum<16>(r);
    r = xor_sum<32>(r);
    if (seg == 0 && mine != 0ull && r < k) K[r] = mine;  // K reused for the winners
  }
  __syncthreads();
}

// Expert id of a top-k key.
MOE_DEV int key_id(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// Where a wave of a gate/up half block reads: lane l's 16 code bytes of K step 4v + i are at
// codes + i * 2048, its four steps' {scale, bias} pairs at the returned sb pointer (see
// gateup_half_block for the lane layout).
MOE_DEV const uint8_t *w13_codes_at(const DecodeArgs &a, int e, int b, int f, int wave, int lane) {
  const size_t blk = (size_t)e * kNB13 + b;
  return a.wt.w13_t + (blk * kNS13 + 4 * wave) * 2048 + (lane >= 32 ? 1024 : 0) + 512 * f +
         16 * (lane & 31);
}
MOE_DEV const uint16_t *w13_sb_at(const DecodeArgs &a, int e, int b, int f, int wave, int lane) {
  const size_t blk = (size_t)e * kNB13 + b;
  return a.wt.w13_tsb + (blk * (kNS13 / 4) + wave) * 512 +
         8 * ((lane >= 32 ? 32 : 0) + 16 * f + ((lane & 31) >> 1));
}

// 16 gate + 16 up rows (rows 32b + 16f .. +16 of expert e's tiled block b) against the
// staged x: wave v takes K steps 4v .. 4v+3, one 1 KB load per step (lanes 0..31 the gate
// rows, 32..63 the up rows; lane: row (l % 32) / 2, K half l % 2). Writes silu(g) * u of
// the 16 rows to hout[0..15]. Called by all DT threads.
MOE_DEV void gateup_half_block(const DecodeArgs &a, int e, int b, int f, const f16x2_t *xs,
                               const float *xseg, float *red, float *hout) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool up = lane >= 32;
  const int r16 = (lane & 31) >> 1, hh = lane & 1;
  const uint8_t *tq = w13_codes_at(a, e, b, f, wave, lane);
  uint4 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = *reinterpret_cast<const uint4 *>(tq + i * 2048);
  const uint4 sb = *reinterpret_cast<const uint4 *>(w13_sb_at(a, e, b, f, wave, lane));
  __syncthreads();  // x staged by the caller
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int st = 4 * wave + i;
    acc += group_dot(dot_codes(c[i], xs, 8 * st + 4 * hh), word_of(sb, i), xseg[2 * st + hh]);
  }
  acc = xor_sum<1>(acc);
  if (hh == 0) red[wave * 32 + (up ? 16 : 0) + r16] = acc;
  __syncthreads();
  if (tid < 16) {
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int v = 0; v < DT / 64; ++v) {
      gs += red[v * 32 + tid];
      us += red[v * 32 + 16 + tid];
    }
    hout[tid] = silu(gs) * us;
  }
}

__global__ __launch_bounds__(DT) void k_dec_a(DecodeArgs a) {
  __shared__ float red[DT / 64];
  const int w = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // router logit w: 512 threads x 4 fp32 weights
  if (w >= a.E) return;
  const float4 wr = reinterpret_cast<const float4 *>(a.router_w + (size_t)w * DH)[tid];
  // the bias leaves with the first loads (a load in a branch here would be waited for
  // only at the end, one more memory latency); without a bias the router row is read and
  // ignored
  const float braw = (a.router_b ? a.router_b : a.router_w)[w];
  const uint2 xb = reinterpret_cast<const uint2 *>(a.x)[tid];
  float xv[4] = {bf16lo(xb.x), bf16hi(xb.x), bf16lo(xb.y), bf16hi(xb.y)};
  if (a.norm) {
    // RMSNorm of the stacked layer's input in fp64, rounded once to bf16: thread t holds
    // elements 4t .. 4t+3, the layout of the RMSNorm kernel, so the bits are the same.
    // Workgroup 0 stores the normalised row for the gate/up kernel.
    __shared__ double red8[DT / 64];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) ss = __builtin_fma((double)xv[i], (double)xv[i], ss);
    const double inv = row_inv_rms_f64(ss, DH, (double)a.eps, red8);
    uint16_t nb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nb[i] = f64_to_bf16_rne((double)xv[i] * inv);
      xv[i] = bf16_to_f32(nb[i]);
    }
    if (w == 0)
      reinterpret_cast<uint2 *>(a.xn)[tid] =
          make_uint2(nb[0] | ((uint32_t)nb[1] << 16), nb[2] | ((uint32_t)nb[3] << 16));
  }
  float d = wr.x * xv[0];
  d = __builtin_fmaf(wr.y, xv[1], d);
  d = __builtin_fmaf(wr.z, xv[2], d);
  d = __builtin_fmaf(wr.w, xv[3], d);
  d = wave_sum_dpp(d);
  if (lane == 0) red[wave] = d;
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < DT / 64; ++i) s += red[i];
    a.z[w] = s + (a.router_b ? braw : 0.f);
  }
}

__global__ __launch_bounds__(DT) void k_dec_b(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint64_t s_key[256];
  __shared__ __attribute__((aligned(16))) uint64_t s_cand[64];
  __shared__ __attribute__((aligned(16))) f16x2_t xs[DH / 2];
  __shared__ float xseg[DH / 32];
  __shared__ float red[DT / 64 * 32];
  const int w = blockIdx.x, tid = threadIdx.x;
  // the logit this thread ranks and its chunk of x leave together
  const int ze = 32 * (tid >> 6) + (tid & 31);
  const float zv = (w < DWG && ze < a.E) ? a.z[ze] : 0.f;
  stage_x(a, xs, xseg);
  if (w >= DWG) {
    // the shared expert needs no routing: half block (b, f) of workgroup DWG + 2b + f
    const int b = (w - DWG) >> 1, f = (w - DWG) & 1;
    gateup_half_block(a, a.E, b, f, xs, xseg, red, a.h + (size_t)a.k * DI + 32 * b + 16 * f);
    return;
  }
  block_topk(zv, a.E, a.k, s_key, s_cand);
  if (w == 0 && tid < a.k) {
    // for C: the winners in rank order, as ids and logits (C forms the softmax weights)
    const uint64_t kw = s_key[tid];
    a.sel_ids[tid] = key_id(kw);
    a.sel_z[tid] = key_float((uint32_t)(kw >> 32));
  }
  const int j = w >> 5, b = (w >> 1) & 15, f = w & 1;
  if (j >= a.k) return;
  gateup_half_block(a, key_id(s_key[j]), b, f, xs, xseg, red,
                    a.h + (size_t)j * DI + 32 * b + 16 * f);
}

// Where lane l reads unit (expert e, K step st) of output rows 64b + 4t .. +4 of the down
// projection (lane: row (l % 8) / 2, K half l % 2): 16 code bytes, and the row's 16-byte
// {scale, bias} entry holding four K steps.
MOE_DEV const uint8_t *w2_codes_at(const DecodeArgs &a, int e, int b, int t, int st, int lane) {
  const size_t blk = (size_t)e * kNB2 + b;
  return a.wt.w2_t + (blk * kNS2 + st) * 2048 + 32 * (4 * t + ((lane & 7) >> 1)) + 16 * (lane & 1);
}
MOE_DEV const uint16_t *w2_sb_at(const DecodeArgs &a, int e, int b, int t, int st, int lane) {
  const size_t blk = (size_t)e * kNB2 + b;
  return a.wt.w2_tsb + (blk * (kNS2 / 4) + (st >> 2)) * 512 + 8 * (4 * t + ((lane & 7) >> 1));
}

__global__ __launch_bounds__(DT) void k_dec_c(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) f16x2_t hs[kSlots * DI / 2];
  __shared__ float hseg[kSlots * DI / 32];
  __shared__ int s_ids[kSlots];
  __shared__ float s_z[kSlots], s_w[kSlots];
  __shared__ float red[DT / 64 * 4];
  const int w = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int k = a.k, nslot = a.k + a.S;
  // token blockIdx.y (the small-T path runs one grid row per token)
  const int tok = blockIdx.y;
  const int32_t *sel_ids = a.sel_ids + (size_t)tok * k;
  const float *sel_z = a.sel_z + (size_t)tok * k;
  const float *hbase = a.h + (size_t)tok * nslot * DI;
  const uint16_t *residual = a.residual ? a.residual + (size_t)tok * DH : nullptr;
  uint16_t *yrow = a.y + (size_t)tok * DH;
  // three independent loads leave together: the routing (ids and logits of the winners),
  // h of all k+1 experts (two 8-element chunks per thread), then -- once the ids are known
  // -- the W2 rows; the routing weights are formed and h is converted into LDS while the W2
  // rows are in flight
  // (the loads are unconditional, with indices clamped into range, so that no branch makes
  // the compiler wait for one before issuing the next)
  const int tq = tid < k ? tid : 0;
  const int my_id = sel_ids[tq];
  const float my_z = sel_z[tq];
  // output rows 64b + 4t .. +4; the residual of row 64b + 4t + tid % 4 (used by threads
  // 0..3; y stands in when there is no residual, read before it is written)
  int b, t;
  down_rows_of(w, b, t);
  const int orow = 64 * b + 4 * t + (tid & 3);
  const uint16_t resid = (residual ? residual : yrow)[orow];
  const int nch = nslot * DI / 8;
  static_assert(kSlots * DI / 8 <= 2 * DT, "h of all slots must fit two chunks per thread");
  float4 hv[2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int ch = min(tid + q * DT, nch - 1);
    hv[q][0] = reinterpret_cast<const float4 *>(hbase)[2 * ch];
    hv[q][1] = reinterpret_cast<const float4 *>(hbase)[2 * ch + 1];
  }
  if (tid < kSlots) {
    s_ids[tid] = tid < k ? min(max(my_id, 0), a.E - 1) : a.E;
    s_z[tid] = my_z;
  }
  __syncthreads();
  // output rows 64b + 4t .. +4; units (slot j, K step s) of 4 rows x 32 code bytes, eight
  // per load instruction: lane group l / 8 takes unit 8p + l / 8; lane: row (l % 8) / 2,
  // K half l % 2
  const int r4 = (lane & 7) >> 1, hh = lane & 1, ug = lane >> 3;
  constexpr int kMaxOcts = (kSlots * kNS2 / 8 + DT / 64 - 1) / (DT / 64);
  uint4 c[kMaxOcts], sb[kMaxOcts];
#pragma unroll
  for (int i = 0; i < kMaxOcts; ++i) {
    // units past the last slot re-read the last slot's rows and go unused: with no branch
    // around the loads, the compiler's wait counts for the later h loads stay exact and
    // these loads stay in flight across the next barrier
    const int p = wave + (DT / 64) * i, u = 8 * p + ug, jj = min(u >> 3, nslot - 1),
              st = u & 7;
    c[i] = *reinterpret_cast<const uint4 *>(w2_codes_at(a, s_ids[jj], b, t, st, lane));
    sb[i] = *reinterpret_cast<const uint4 *>(w2_sb_at(a, s_ids[jj], b, t, st, lane));
  }
  // routing weights: softmax over the selected logits, s_z[0] the largest (or, on the
  // small-T path, the weights themselves); the shared expert (slot k) has weight 1
  if (tid < kSlots) {
    float wj = 1.0f;
    if (tid < k && a.sel_is_w) {
      wj = s_z[tid];
    } else if (tid < k) {
      const float top = s_z[0];
      float den = 0.f, mine = 0.f;
#pragma unroll
      for (int q = 0; q < kMaxTopK; ++q) {
        if (q < k) {
          // exp(z - top) from the hardware exp2; top == -inf only when every logit is -inf
          const float ex = top == -INFINITY
                               ? 1.0f
                               : __builtin_amdgcn_exp2f((s_z[q] - top) * 1.4426950408889634f);
          den += ex;
          if (q == tid) mine = ex;
        }
      }
      wj = mine / den;
    }
    s_w[tid] = wj;
  }
  // h -> fp16 pairs (v[8c + p], v[8c + p + 4]) per chunk c, and the 32-element segment sums
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int ch = tid + q * DT;
    const bool live = ch < nch;
    const float v[8] = {hv[q][0].x, hv[q][0].y, hv[q][0].z, hv[q][0].w,
                        hv[q][1].x, hv[q][1].y, hv[q][1].z, hv[q][1].w};
    float sum = 0.f;
    f16x2_t pr[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      pr[pp] = live ? f16x2_t{(_Float16)v[pp], (_Float16)v[pp + 4]} : f16x2_t{};
      sum += (float)pr[pp][0] + (float)pr[pp][1];
    }
    if (live) *reinterpret_cast<uint4 *>(hs + 4 * ch) = __builtin_bit_cast(uint4, pr);
    sum = xor_sum<1>(sum);
    sum = xor_sum<2>(sum);
    if ((ch & 3) == 0 && live) hseg[ch >> 2] = sum;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxOcts; ++i) {
    const int p = wave + (DT / 64) * i, u = 8 * p + ug, jj = u >> 3, st = u & 7;
    if (jj < nslot) {
      const float raw = dot_codes(c[i], hs + jj * (DI / 2), 8 * st + 4 * hh);
      acc = __builtin_fmaf(s_w[jj], group_dot(raw, word_of(sb[i], st & 3),
                                               hseg[jj * (DI / 32) + 2 * st + hh]), acc);
    }
  }
  // lanes of one row: both K halves (xor 1) and the eight unit groups (xor 8, 16, 32)
  acc = xor_sum<1>(acc);
  acc = xor_sum<8>(acc);
  acc = xor_sum<16>(acc);
  acc = xor_sum<32>(acc);
  if (lane < 8 && hh == 0) red[wave * 4 + r4] = acc;
  __syncthreads();
  if (tid < 4) {
    float y = 0.f;
#pragma unroll
    for (int v = 0; v < DT / 64; ++v) y += red[v * 4 + tid];
    if (residual) y += bf16_to_f32(resid);
    yrow[orow] = f32_to_bf16(y);
  }
}

// ---- small-T path: 2 <= T <= kSmallT tokens of one layer, three kernels like decode -------
// Section "Optimize the one-row weight path" carried to a few rows: each selected expert's
// weights are read once for all the tokens that chose it, so the bytes grow with the union
// of the tokens' experts, not with T. The prefill pipeline (routing tables, tile map,
// grouped GEMMs, combine) costs a fixed ~60 us at such T.
//   SA  one workgroup per expert e: router row e read once, dot products with every token.
//   SB  every workgroup redoes the T top-k's (wave t takes token t), builds the union of the
//       selected experts (ascending id, plus the shared expert) with a token mask per
//       expert, then walks units (expert, 16 gate + 16 up rows) w, w + 256, ...: one load of
//       the unit's codes serves every token in its mask. h[t][j] lands in the slot j of the
//       expert in token t's ascending id list (the shared expert in slot k).
//   SC  the decode output kernel, one grid row per token, with the weights from SB.

// SA: z[t][e] for the T tokens; thread i holds router weights 4i .. 4i+3.
__global__ __launch_bounds__(DT) void k_st_a(DecodeArgs a) {
  __shared__ float red[kSmallT][DT / 64];
  const int e = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int T = a.T;
  // every load leaves before the first use (tokens past T re-read the last one)
  const float4 wr = reinterpret_cast<const float4 *>(a.router_w + (size_t)e * DH)[tid];
  const float braw = (a.router_b ? a.router_b : a.router_w)[e];
  uint2 xb[kSmallT];
#pragma unroll
  for (int i = 0; i < kSmallT; ++i)
    xb[i] = reinterpret_cast<const uint2 *>(a.x + (size_t)min(i, T - 1) * DH)[tid];
#pragma unroll
  for (int i = 0; i < kSmallT; ++i) {
    if (i < T) {
      float d = wr.x * bf16lo(xb[i].x);
      d = __builtin_fmaf(wr.y, bf16hi(xb[i].x), d);
      d = __builtin_fmaf(wr.z, bf16lo(xb[i].y), d);
      d = __builtin_fmaf(wr.w, bf16hi(xb[i].y), d);
      d = wave_sum_dpp(d);
      if (lane == 0) red[i][wave] = d;
    }
  }
  __syncthreads();
  if (tid < T) {
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < DT / 64; ++v) s += red[tid][v];
    a.z[(size_t)tid * a.E + e] = s + (a.router_b ? braw : 0.f);
  }
}

// SB: top-k of every token, the union of their experts, then the gate/up units.
__global__ __launch_bounds__(DT) void k_st_b(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) f16x2_t xs[kSmallT][DH / 2];
  __shared__ float xseg[kSmallT][DH / 32];
  __shared__ __attribute__((aligned(16))) uint64_t s_topk[kSmallT][kTopkScratch];
  __shared__ int s_list[kMaxExperts + 1];
  __shared__ uint32_t s_mask[kMaxExperts + 1], s_jtab[kMaxExperts + 1];
  __shared__ uint32_t m_raw[kMaxExperts], jt_raw[kMaxExperts];
  __shared__ int s_wtot[4];
  __shared__ float red[2][kSmallT][DT / 64 * 32];
  const int w = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int T = a.T, E = a.E, k = a.k;
  // loads: wave t's token logits (lane l: experts l, l+64, l+128, l+192; past E the last
  // expert, masked by the top-k) and every token's x (chunk ch = tid + DT q of the T x 256
  // chunks; past them the last chunk again, not stored)
  const int tw = min(wave, T - 1);
  float zv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) zv[c] = a.z[(size_t)tw * E + min(lane + 64 * c, E - 1)];
  constexpr int kXQ = kSmallT * (DH / 8) / DT;
  uint4 xr[kXQ];
#pragma unroll
  for (int q = 0; q < kXQ; ++q) {
    const int ch = min(tid + DT * q, T * (DH / 8) - 1);
    xr[q] = reinterpret_cast<const uint4 *>(a.x)[ch];
  }
  // x -> fp16 pairs (v[8c + p], v[8c + p + 4]) and 32-element segment sums, per token
#pragma unroll
  for (int q = 0; q < kXQ; ++q) {
    const int ch = tid + DT * q;
    const bool live = ch < T * (DH / 8);
    const int ti = ch / (DH / 8), c = ch % (DH / 8);
    const uint32_t wd[4] = {xr[q].x, xr[q].y, xr[q].z, xr[q].w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16lo(wd[i]);
      v[2 * i + 1] = bf16hi(wd[i]);
    }
    float sum = 0.f;
    f16x2_t pr[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      pr[pp] = f16x2_t{(_Float16)v[pp], (_Float16)v[pp + 4]};
      sum += (float)pr[pp][0] + (float)pr[pp][1];
    }
    if (live) *reinterpret_cast<uint4 *>(&xs[ti][4 * c]) = __builtin_bit_cast(uint4, pr);
    sum = xor_sum<1>(sum);
    sum = xor_sum<2>(sum);
    if ((c & 3) == 0 && live) xseg[ti][c >> 2] = sum;
  }
  if (tid < kMaxExperts) m_raw[tid] = jt_raw[tid] = 0;
  __syncthreads();
  // top-k: wave t < T takes token t (ids in ascending order, weights from the softmax);
  // each winner marks its expert with the token's bit and its slot (LDS bitwise ORs, so
  // the result does not depend on their order)
  if (wave < T) {
    int id, pos;
    float wt;
    wave_topk(zv, E, k, s_topk[wave], id, pos, wt);
    if (lane < k) {
      atomicOr(&m_raw[id], 1u << wave);
      atomicOr(&jt_raw[id], (uint32_t)pos << (4 * wave));
      if (w == 0) {
        a.sel_ids[(size_t)wave * k + pos] = id;
        a.sel_z[(size_t)wave * k + pos] = wt;
      }
    }
  }
  __syncthreads();
  // the union: expert e's token mask and its slot in each token's list (4 bits per
  // token); a workgroup scan packs the chosen experts in ascending id order (after the
  // shared expert)
  const uint32_t mask = tid < kMaxExperts ? m_raw[tid] : 0u;
  const uint32_t jt = tid < kMaxExperts ? jt_raw[tid] : 0u;
  const bool nz = tid < kMaxExperts && mask != 0;
  const uint64_t bal = __ballot(nz);
  const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
  if (lane == 0 && wave < 4) s_wtot[wave] = __popcll(bal);
  __syncthreads();
  int base = 0, nu = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    base += v < wave ? s_wtot[v] : 0;
    nu += s_wtot[v];
  }
  // the shared expert (every token, slot k) comes first: its units carry all T tokens, so
  // they start with everyone else's first units instead of trailing at the end
  const int sh = a.S;
  if (nz) {
    s_list[sh + base + before] = tid;
    s_mask[sh + base + before] = mask;
    s_jtab[sh + base + before] = jt;
  }
  if (tid == 0 && sh) {
    s_list[0] = E;
    s_mask[0] = (1u << T) - 1;
    uint32_t all = 0;
    for (int t = 0; t < T; ++t) all |= (uint32_t)k << (4 * t);
    s_jtab[0] = all;
  }
  __syncthreads();
  const int nunits = (nu + a.S) * (2 * kNB13);
  // units u = w, w + G, ...: expert u / 32, W13 block (u / 2) % 16, half u % 2; wave v takes
  // K steps 4v .. 4v+3 of the unit's 32 rows (lanes 0..31 gate rows, 32..63 up rows; lane:
  // row (l % 32) / 2, K half l % 2), as in the decode kernel.
  const bool up = lane >= 32;
  const int r16 = (lane & 31) >> 1, hh = lane & 1;
  struct Unit {
    uint4 c0, c1, c2, c3, sb;
  };
  auto unit_load = [&](int u) {
    const int ex = u >> 5, b = (u >> 1) & 15, f = u & 1;
    const size_t blk = (size_t)s_list[ex] * kNB13 + b;
    const uint8_t *tq = a.wt.w13_t + (blk * kNS13 + 4 * wave) * 2048 + (up ? 1024 : 0) +
                        512 * f + 16 * (lane & 31);
    Unit d;
    d.c0 = *reinterpret_cast<const uint4 *>(tq);
    d.c1 = *reinterpret_cast<const uint4 *>(tq + 2048);
    d.c2 = *reinterpret_cast<const uint4 *>(tq + 2 * 2048);
    d.c3 = *reinterpret_cast<const uint4 *>(tq + 3 * 2048);
    d.sb = *reinterpret_cast<const uint4 *>(
        a.wt.w13_tsb + (blk * (kNS13 / 4) + wave) * 512 + 8 * ((up ? 32 : 0) + 16 * f + r16));
    return d;
  };
  int par = 0;
  auto unit_compute = [&](int u, const Unit &d) {
    const int ex = u >> 5, b = (u >> 1) & 15, f = u & 1;
    const uint32_t m = s_mask[ex], jt = s_jtab[ex];
    const uint4 cc[4] = {d.c0, d.c1, d.c2, d.c3};
#pragma unroll 1
    for (int t = 0; t < kSmallT; ++t) {
      if ((m >> t) & 1) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int st = 4 * wave + i;
          acc += group_dot(dot_codes(cc[i], xs[t], 8 * st + 4 * hh), word_of(d.sb, i),
                           xseg[t][2 * st + hh]);
        }
        acc = xor_sum<1>(acc);
        if (hh == 0) red[par][t][wave * 32 + (up ? 16 : 0) + r16] = acc;
      }
    }
    __syncthreads();
    const int t = tid >> 4, r = tid & 15;
    if (t < kSmallT && ((m >> t) & 1)) {
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int v = 0; v < DT / 64; ++v) {
        gs += red[par][t][v * 32 + r];
        us += red[par][t][v * 32 + 16 + r];
      }
      const int j = (jt >> (4 * t)) & 15;
      a.h[((size_t)t * (k + a.S) + j) * DI + 32 * b + 16 * f + r] = silu(gs) * us;
    }
    par ^= 1;
  };
  // units run two ahead: while unit u computes, the loads of units u + G and u + 2G are in
  // flight (past the last unit the last one is loaded again, unused). Three register sets,
  // each reloaded right after its unit is computed, so no set is ever copied (a copy would
  // wait for its loads).
  const int G = gridDim.x, last = nunits - 1;
  Unit d0 = unit_load(min(w, last)), d1 = unit_load(min(w + G, last)),
       d2 = unit_load(min(w + 2 * G, last));
  for (int u = w; u < nunits; u += 3 * G) {
    unit_compute(u, d0);
    d0 = unit_load(min(u + 3 * G, last));
    if (u + G < nunits) unit_compute(u + G, d1);
    d1 = unit_load(min(u + 4 * G, last));
    if (u + 2 * G < nunits) unit_compute(u + 2 * G, d2);
    d2 = unit_load(min(u + 5 * G, last));
  }
}

// ---- weight-read ceilings (measurement aids) ----------------------------------------------
// Each kernel issues exactly the weight loads of one decode kernel, from the same grid and
// addresses (the helpers above), with the arithmetic taken out: a thread only XORs the words
// it read and stores the result when it equals a fixed word (practically never), so the loads
// cannot be dropped. The selected experts come from a.sel_ids (k ids) and the shared expert.
// Timed beside the product kernels they give the fastest rate of the same access pattern.
MOE_DEV uint32_t xor4(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }
constexpr uint32_t kSinkWord = 0x9E3779B9u;

__global__ __launch_bounds__(DT) void k_read_router(DecodeArgs a, uint32_t *sink) {
  const int w = blockIdx.x, tid = threadIdx.x;
  if (w >= a.E) return;
  const uint4 wr = reinterpret_cast<const uint4 *>(a.router_w + (size_t)w * DH)[tid];
  const uint2 xb = reinterpret_cast<const uint2 *>(a.x)[tid];
  const uint32_t v = xor4(wr) ^ xb.x ^ xb.y;
  if (v == kSinkWord) sink[0] = v;
}

__global__ __launch_bounds__(DT) void k_read_gateup(DecodeArgs a, uint32_t *sink) {
  const int w = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int e, b, f;
  if (w >= DWG) {
    e = a.E;
    b = (w - DWG) >> 1;
    f = (w - DWG) & 1;
  } else {
    const int j = w >> 5;
    if (j >= a.k) return;
    e = a.sel_ids[j];
    b = (w >> 1) & 15;
    f = w & 1;
  }
  const uint8_t *tq = w13_codes_at(a, e, b, f, wave, lane);
  uint32_t v = xor4(*reinterpret_cast<const uint4 *>(w13_sb_at(a, e, b, f, wave, lane)));
#pragma unroll
  for (int i = 0; i < 4; ++i) v ^= xor4(*reinterpret_cast<const uint4 *>(tq + i * 2048));
  if (v == kSinkWord) sink[0] = v;
}

__global__ __launch_bounds__(DT) void k_read_down(DecodeArgs a, uint32_t *sink) {
  const int w = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nslot = a.k + a.S, ug = lane >> 3;
  int b, t;
  down_rows_of(w, b, t);
  uint32_t v = 0;
  constexpr int kMaxOcts = (kSlots * kNS2 / 8 + DT / 64 - 1) / (DT / 64);
#pragma unroll
  for (int i = 0; i < kMaxOcts; ++i) {
    const int u = 8 * (wave + (DT / 64) * i) + ug, jj = u >> 3, st = u & 7;
    if (jj < nslot) {  // only the units the product kernel uses
      const int e = jj < a.k ? a.sel_ids[jj] : a.E;
      v ^= xor4(*reinterpret_cast<const uint4 *>(w2_codes_at(a, e, b, t, st, lane)));
      v ^= xor4(*reinterpret_cast<const uint4 *>(w2_sb_at(a, e, b, t, st, lane)));
    }
  }
  if (v == kSinkWord) sink[0] = v;
}

hipError_t launch_read_ceiling(const DecodeArgs &a, int part, uint32_t *sink, hipStream_t s) {
  if (part == 0)
    MOE_LAUNCH("k_read_router", k_read_router, dim3(DWG), dim3(DT), 0, s, a, sink);
  else if (part == 1)
    MOE_LAUNCH("k_read_gateup", k_read_gateup, dim3(DWG + (a.S ? kSharedWG : 0)), dim3(DT), 0, s,
               a, sink);
  else
    MOE_LAUNCH("k_read_down", k_read_down, dim3(kDownWG), dim3(DT), 0, s, a, sink);
  return hipSuccess;
}

bool decode_gemv_supported(int H, int I, int E, int k, int S, bool int4) {
  return int4 && H == DH && I == DI && E <= 256 && k + S <= kSlots;
}

hipError_t launch_small_t(const DecodeArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_st_a", k_st_a, dim3(a.E), dim3(DT), 0, s, a);
  MOE_LAUNCH("k_st_b", k_st_b, dim3(DWG), dim3(DT), 0, s, a);
  MOE_LAUNCH("k_dec_c", k_dec_c, dim3(kDownWG, a.T), dim3(DT), 0, s, a);
  return hipSuccess;
}

hipError_t launch_decode_gemv(const DecodeArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_dec_a", k_dec_a, dim3(DWG), dim3(DT), 0, s, a);
  MOE_LAUNCH("k_dec_b", k_dec_b, dim3(DWG + (a.S ? kSharedWG : 0)), dim3(DT), 0, s, a);
  MOE_LAUNCH("k_dec_c", k_dec_c, dim3(kDownWG), dim3(DT), 0, s, a);
  return hipSuccess;
}

}  // namespace moe
