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
constexpr int kGdnLanes = 16;   // lanes per state row (32 measured slower: one more reduction step)

// sum over the L lanes of an aligned group (xor 16 by permlane swap, the rest by DPP; the
// rotation by 4 stands for xor 4 right after the xor-8 step)
template <int L>
MOE_DEV float group_sum_dpp(float v) {
  if constexpr (L == 32) v = xor_sum<16>(v);
  v = xor_sum<8>(v);
  v = xor_sum<4>(v);
  v = xor_sum<2>(v);
  return xor_sum<1>(v);
}
}  // namespace

// L lanes per state row (EL = 128 / L values each), 64 / L rows per wave, RW rows per
// workgroup of four waves; grid (value heads, 128 / RW). Workgroup ids are dealt over the 8
// XCDs round-robin, so with the head as the fast grid index all row blocks of a head run on
// one XCD and its q and k are fetched into that XCD's L2 once (head-major order put them
// on eight XCDs and read the inputs about four times over from memory).
template <int L>
__global__ __launch_bounds__(256, 1) void k_gdn_scan(GdnArgs a) {
  constexpr int D = kGdnD, C = kGdnChunk, EL = D / L, RW = 4 * (64 / L);
  const int j = blockIdx.x, i0 = blockIdx.y * RW;
  const int kh = j / (a.n_v / a.n_k);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane / L, lr = lane % L;
  const int rl = wave * (64 / L) + g;  // this lane group's row inside the workgroup

  __shared__ __attribute__((aligned(16))) float sK[C][D];
  __shared__ __attribute__((aligned(16))) float sQ[C][D];
  __shared__ float sV[C][RW];
  __shared__ __attribute__((aligned(16))) float4 sS[C];  // alpha, beta, k . q, alpha beta
  __shared__ __attribute__((aligned(16))) uint16_t sO[C][RW];

  // the row's state, EL values at d = EL lr .. +EL
  float *srow = a.state + ((size_t)j * D + i0 + rl) * D + EL * lr;
  float s[EL];
#pragma unroll
  for (int e = 0; e < EL; e += 4) {
    const float4 x = *reinterpret_cast<const float4 *>(srow + e);
    s[e] = x.x; s[e + 1] = x.y; s[e + 2] = x.z; s[e + 3] = x.w;
  }

  // staging registers of one block: q and k (4 x 16 bytes each per thread), the block's v
  // slice (threads 0 .. 8 RW - 1: one 16-byte piece each), alpha (128..191), beta (192..255)
  constexpr int VT = C * RW / 8;  // threads holding v
  uint4 rq[4], rk[4], rv = {0, 0, 0, 0};
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
    if (tid < VT) {
      const int tt = tid / (RW / 8), part = tid % (RW / 8);
      const int64_t t = t0 + tt < a.T ? t0 + tt : a.T - 1;
      rv = *reinterpret_cast<const uint4 *>(a.v + ((size_t)t * a.n_v + j) * D + i0 + 8 * part);
    } else if (tid >= 128) {
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
    if (tid < VT) {
      widen(rv, &sV[tid / (RW / 8)][8 * (tid % (RW / 8))]);
    } else if (tid >= 128) {
      reinterpret_cast<float *>(&sS[(tid - 128) & 63])[tid < 192 ? 0 : 1] = rab;
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
      if (part == 0) {
        float *sc = reinterpret_cast<float *>(&sS[tt]);
        sc[2] = p;
        sc[3] = sc[0] * sc[1];
      }
    }
    __syncthreads();
    if (c + 1 < nch) fetch(t0 + C);  // in flight while this block is scanned

    // Token tt + 1's operands are requested from LDS before token tt's dependent chain
    // runs (two register sets in turn, indices clamped so every read is unconditional):
    // one LDS round trip per token is hidden behind the chain instead of three waited on.
    struct Tok {
      float kv[EL], qv[EL];
      float4 sc;  // alpha, beta, k . q, alpha beta
      float vr;
    };
    auto ld = [&](int tt) {
      Tok t;
#pragma unroll
      for (int e = 0; e < EL; e += 4) {
        const float4 k4 = *reinterpret_cast<const float4 *>(&sK[tt][EL * lr + e]);
        const float4 q4 = *reinterpret_cast<const float4 *>(&sQ[tt][EL * lr + e]);
        t.kv[e] = k4.x; t.kv[e + 1] = k4.y; t.kv[e + 2] = k4.z; t.kv[e + 3] = k4.w;
        t.qv[e] = q4.x; t.qv[e + 1] = q4.y; t.qv[e + 2] = q4.z; t.qv[e + 3] = q4.w;
      }
      t.sc = sS[tt];
      t.vr = sV[tt][rl];
      return t;
    };
    auto step = [&](const Tok &t, int tt) {
      float pb0 = s[0] * t.kv[0], pb1 = s[1] * t.kv[1];
      float pa0 = s[0] * t.qv[0], pa1 = s[1] * t.qv[1];
#pragma unroll
      for (int e = 2; e < EL; e += 2) {
        pb0 = __builtin_fmaf(s[e], t.kv[e], pb0);
        pb1 = __builtin_fmaf(s[e + 1], t.kv[e + 1], pb1);
        pa0 = __builtin_fmaf(s[e], t.qv[e], pa0);
        pa1 = __builtin_fmaf(s[e + 1], t.qv[e + 1], pa1);
      }
      const float b = group_sum_dpp<L>(pb0 + pb1);
      const float av = group_sum_dpp<L>(pa0 + pa1);
      const float cc = __builtin_fmaf(-t.sc.w, b, t.sc.y * t.vr);  // beta (v - alpha b)
      const float o = __builtin_fmaf(t.sc.x, av, cc * t.sc.z);
#pragma unroll
      for (int e = 0; e < EL; ++e) s[e] = __builtin_fmaf(cc, t.kv[e], t.sc.x * s[e]);
      sO[tt][rl] = f32_to_bf16(o);  // every lane of the row stores the same value
    };
    // Both steps of a pair run unconditionally (a load under a branch is waited for where
    // the branch joins): a token past the block's end gets alpha = 1, beta = 0, which leaves
    // the state exactly as it is, and its output lands in an unused row of the staging.
    // (the scheduling barriers keep the next token's reads ahead of the current chain; left
    // alone, the scheduler issues them halfway through it, too late to hide their latency)
    Tok ta = ld(0);
    for (int tt = 0; tt < nt; tt += 2) {
      Tok tb = ld(tt + 1 < C ? tt + 1 : C - 1);
      __builtin_amdgcn_sched_barrier(0);
      step(ta, tt);
      ta = ld(tt + 2 < C ? tt + 2 : C - 1);
      __builtin_amdgcn_sched_barrier(0);
      if (tt + 1 >= nt) tb.sc = float4{1.f, 0.f, 0.f, 0.f};  // alpha 1, beta 0
      step(tb, tt + 1 < C ? tt + 1 : C - 1);
    }
    __syncthreads();
    // the block's outputs: per token, this workgroup's RW rows are contiguous
    if (tid < nt * (RW / 8)) {
      const int tt = tid / (RW / 8), h = tid % (RW / 8);
      *reinterpret_cast<uint4 *>(a.out + ((size_t)(t0 + tt) * a.n_v + j) * D + i0 + 8 * h) =
          *reinterpret_cast<const uint4 *>(&sO[tt][8 * h]);
    }
  }
#pragma unroll
  for (int e = 0; e < EL; e += 4)
    *reinterpret_cast<float4 *>(srow + e) = float4{s[e], s[e + 1], s[e + 2], s[e + 3]};
}

// ---- chunked form ------------------------------------------------------------------------
// Tokens in chunks of 32 (r = 0..31 inside a chunk, S the state before it). The gate
// products R[i][r] = prod_{i<j<=r} alpha_j (R[r][r] = 1) and gam_r = prod_{j<=r} alpha_j are
// formed as products, never as ratios. With G[i][r] = k_i . k_r and M[i][r] = k_i . q_r:
//   W_r = beta_r (k_r - sum_{i<r} G[i][r] W_i)                (the WY factors of prod (I - b k k^T))
//   U_r = beta_r (v_r - sum_{i<r} R[i][r] G[i][r] U_i)
// and then, per state row s (a row of S):
//   P_i = s . W_i,  Qs_r = s . q_r
//   o_r = gam_r (Qs_r - sum_{i<=r} M[i][r] P_i) + sum_{i<=r} R[i][r] M[i][r] U_i[row]
//   s  <- gam_31 s + sum_i (R[i][31] U_i[row] - gam_31 P_i) k_i
// W, U and the chunk's coefficient tables depend on the inputs only, so k_gdn_prep forms
// them for every chunk at once; k_gdn_chunks then walks the chunks in order with the state
// in registers. Tokens past the end get alpha = 1, beta = 0 and zero q, k, v.
namespace {
constexpr int kCk = 32;                                 // tokens per chunk
constexpr int kCkFloats = 2 * kCk * kGdnD + 2 * kCk * kCk + 2 * kCk;  // per (head, chunk)
constexpr int kPad = kGdnD + 4;                          // LDS row stride (bank spread)
}  // namespace

size_t gdn_chunk_ws_bytes(int64_t T, int n_v) {
  return (size_t)((T + kCk - 1) / kCk) * n_v * kCkFloats * 4;
}

// one workgroup per (value head, chunk): W, U, A1 = M (i <= r), A2 = R M (i <= r),
// e_i = R[i][31], gam_r
__global__ __launch_bounds__(256) void k_gdn_prep(GdnArgs a) {
  constexpr int D = kGdnD, C = kCk;
  const int j = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int kh = j / (a.n_v / a.n_k);
  const int64_t t0 = (int64_t)c * C;
  __shared__ __attribute__((aligned(16))) float sK[C][kPad];
  __shared__ __attribute__((aligned(16))) float sQ[C][kPad];
  __shared__ __attribute__((aligned(16))) float sV[C][kPad];
  __shared__ float sG[C][C + 1], sM[C][C + 1], sR[C][C + 1], sGU[C][C + 1];
  __shared__ float sAl[C], sBe[C], sGam[C];
  // inputs: 32 rows x 16 pieces of 8 values for each of q, k, v
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int f = tid + 256 * i, r = f >> 4, part = f & 15;
    const int64_t t = t0 + r;
    uint4 uq = {0, 0, 0, 0}, uk = {0, 0, 0, 0}, uv = {0, 0, 0, 0};
    if (t < a.T) {
      const size_t off = ((size_t)t * a.n_k + kh) * D + 8 * part;
      uq = *reinterpret_cast<const uint4 *>(a.q + off);
      uk = *reinterpret_cast<const uint4 *>(a.k + off);
      uv = *reinterpret_cast<const uint4 *>(a.v + ((size_t)t * a.n_v + j) * D + 8 * part);
    }
    const uint32_t wq[4] = {uq.x, uq.y, uq.z, uq.w}, wk[4] = {uk.x, uk.y, uk.z, uk.w},
                   wv[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sQ[r][8 * part + 2 * e] = bf16lo(wq[e]);
      sQ[r][8 * part + 2 * e + 1] = bf16hi(wq[e]);
      sK[r][8 * part + 2 * e] = bf16lo(wk[e]);
      sK[r][8 * part + 2 * e + 1] = bf16hi(wk[e]);
      sV[r][8 * part + 2 * e] = bf16lo(wv[e]);
      sV[r][8 * part + 2 * e + 1] = bf16hi(wv[e]);
    }
  }
  if (tid < C) {
    const int64_t t = t0 + tid;
    sAl[tid] = t < a.T ? a.alpha[(size_t)t * a.n_v + j] : 1.f;
    sBe[tid] = t < a.T ? a.beta[(size_t)t * a.n_v + j] : 0.f;
  }
  __syncthreads();
  // G and M: 2 x 32 x 32 dot products of 128, eight per thread
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int d = tid + 256 * m, which = d >> 10, i = (d >> 5) & 31, r = d & 31;
    const float4 *x = reinterpret_cast<const float4 *>(sK[i]);
    const float4 *y = reinterpret_cast<const float4 *>(which ? sQ[r] : sK[r]);
    float p0 = 0.f, p1 = 0.f;
#pragma unroll 8
    for (int e = 0; e < D / 4; ++e) {
      const float4 u = x[e], w = y[e];
      p0 = __builtin_fmaf(u.x, w.x, p0);
      p1 = __builtin_fmaf(u.y, w.y, p1);
      p0 = __builtin_fmaf(u.z, w.z, p0);
      p1 = __builtin_fmaf(u.w, w.w, p1);
    }
    (which ? sM : sG)[i][r] = p0 + p1;
  }
  // gate products: R[i][r] for r >= i (zero below), gam_r
  if (tid < C) {
    float run = 1.f;
    for (int r = 0; r < C; ++r) {
      if (r > tid) run *= sAl[r];
      sR[tid][r] = r >= tid ? run : 0.f;
    }
  } else if (tid == C) {
    float g = 1.f;
    for (int r = 0; r < C; ++r) {
      g *= sAl[r];
      sGam[r] = g;
    }
  }
  __syncthreads();
  for (int f = tid; f < C * C; f += 256) sGU[f >> 5][f & 31] = sR[f >> 5][f & 31] * sG[f >> 5][f & 31];
  __syncthreads();
  float *ws = a.ws + ((size_t)j * a.nch + c) * kCkFloats;
  {
    // forward substitution, one column per thread: W (threads 0..127), U (128..255)
    const int col = tid & 127, isU = tid >> 7;
    float x[C];
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float acc = isU ? sV[r][col] : sK[r][col];
#pragma unroll
      for (int i = 0; i < r; ++i) {
        const float g = isU ? sGU[i][r] : sG[i][r];
        acc = __builtin_fmaf(-g, x[i], acc);
      }
      x[r] = sBe[r] * acc;
    }
    float *dst = ws + (isU ? C * D : 0) + col;
#pragma unroll
    for (int r = 0; r < C; ++r) dst[r * D] = x[r];
  }
  // coefficient tables, token-major: A1[r][i] = M[i][r], A2[r][i] = R[i][r] M[i][r] (i <= r)
  float *A1 = ws + 2 * C * D, *A2 = A1 + C * C, *E = A2 + C * C, *Gm = E + C;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int f = tid + 256 * m, r = f >> 5, i = f & 31;
    const float mm = i <= r ? sM[i][r] : 0.f;
    A1[f] = mm;
    A2[f] = mm * sR[i][r];
  }
  if (tid < C) {
    E[tid] = sR[tid][C - 1];
    Gm[tid] = sGam[tid];
  }
}

// grid (value heads, 8 row slices of 16), the chunks in order; layout of the register scan
// (one state row per 16-lane DPP row, 8 values per lane)
__global__ __launch_bounds__(256, 1) void k_gdn_chunks(GdnArgs a) {
  constexpr int D = kGdnD, C = kCk, R = 16, EL = 8;
  const int j = blockIdx.x, i0 = blockIdx.y * R;
  const int kh = j / (a.n_v / a.n_k);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, lr = lane & 15;
  const int rl = wave * 4 + g;  // state row of this lane group

  __shared__ __attribute__((aligned(16))) float sW[C][kPad];
  __shared__ __attribute__((aligned(16))) float sQ[C][kPad];
  __shared__ __attribute__((aligned(16))) float sK[C][kPad];
  __shared__ __attribute__((aligned(16))) float sU[R][C + 4];    // U_i[row], row-major
  __shared__ __attribute__((aligned(16))) float sA1[C][C + 4];   // [r][i]
  __shared__ __attribute__((aligned(16))) float sA2[C][C + 4];
  __shared__ __attribute__((aligned(16))) float sP[R][C + 4];    // P_i of each row
  __shared__ __attribute__((aligned(16))) float sQs[R][C + 4];   // Qs_r of each row
  __shared__ __attribute__((aligned(16))) float sE[C];
  __shared__ float sGm[C];
  __shared__ __attribute__((aligned(16))) uint16_t sO[C][R];

  float *srow = a.state + ((size_t)j * D + i0 + rl) * D + EL * lr;
  float s[EL];
  {
    const float4 x = *reinterpret_cast<const float4 *>(srow);
    const float4 y = *reinterpret_cast<const float4 *>(srow + 4);
    s[0] = x.x; s[1] = x.y; s[2] = x.z; s[3] = x.w;
    s[4] = y.x; s[5] = y.y; s[6] = y.z; s[7] = y.w;
  }
  // staging registers of one chunk (loaded a chunk ahead, stored to LDS after the scan)
  float4 rW0, rW1, rW2, rW3, rA1, rA2, rU;  // named, not an array (an array went to scratch)
  uint4 rq[2], rk[2];
  float rEG = 0.f;
  auto fetch = [&](int c) {
    const float *ws = a.ws + ((size_t)j * a.nch + c) * kCkFloats;
    const int64_t t0 = (int64_t)c * C;
    auto ldw = [&](int m) {
      const int f = tid + 256 * m, r = f >> 5, part = f & 31;
      return *reinterpret_cast<const float4 *>(ws + r * D + 4 * part);
    };
    rW0 = ldw(0);
    rW1 = ldw(1);
    rW2 = ldw(2);
    rW3 = ldw(3);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int f = tid + 256 * m, r = f >> 4, part = f & 15;
      const int64_t t = t0 + r < a.T ? t0 + r : a.T - 1;
      const size_t off = ((size_t)t * a.n_k + kh) * D + 8 * part;
      rq[m] = *reinterpret_cast<const uint4 *>(a.q + off);
      rk[m] = *reinterpret_cast<const uint4 *>(a.k + off);
    }
    rA1 = *reinterpret_cast<const float4 *>(ws + 2 * C * D + 4 * tid);
    rA2 = *reinterpret_cast<const float4 *>(ws + 2 * C * D + C * C + 4 * tid);
    {
      // U_i[i0 .. i0+15] for the 32 tokens: 128 pieces of 4 (threads 0..127)
      const int i = (tid & 127) >> 2, part = tid & 3;
      rU = *reinterpret_cast<const float4 *>(ws + C * D + i * D + i0 + 4 * part);
    }
    if (tid < 2 * C) rEG = ws[2 * C * D + 2 * C * C + tid];
  };
  auto stage = [&]() {
    auto stw = [&](int m, float4 w) {
      const int f = tid + 256 * m, r = f >> 5, part = f & 31;
      *reinterpret_cast<float4 *>(&sW[r][4 * part]) = w;
    };
    stw(0, rW0);
    stw(1, rW1);
    stw(2, rW2);
    stw(3, rW3);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int f = tid + 256 * m, r = f >> 4, part = f & 15;
      const uint32_t wq[4] = {rq[m].x, rq[m].y, rq[m].z, rq[m].w};
      const uint32_t wk[4] = {rk[m].x, rk[m].y, rk[m].z, rk[m].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sQ[r][8 * part + 2 * e] = bf16lo(wq[e]);
        sQ[r][8 * part + 2 * e + 1] = bf16hi(wq[e]);
        sK[r][8 * part + 2 * e] = bf16lo(wk[e]);
        sK[r][8 * part + 2 * e + 1] = bf16hi(wk[e]);
      }
    }
    *reinterpret_cast<float4 *>(&sA1[tid >> 3][4 * (tid & 7)]) = rA1;
    *reinterpret_cast<float4 *>(&sA2[tid >> 3][4 * (tid & 7)]) = rA2;
    if (tid < 128) {
      const int i = tid >> 2, part = tid & 3;
      sU[4 * part][i] = rU.x;
      sU[4 * part + 1][i] = rU.y;
      sU[4 * part + 2][i] = rU.z;
      sU[4 * part + 3][i] = rU.w;
    }
    if (tid < C) sE[tid] = rEG;
    else if (tid < 2 * C) sGm[tid - C] = rEG;
  };

  fetch(0);
  for (int c = 0; c < a.nch; ++c) {
    const int64_t t0 = (int64_t)c * C;
    const int n = (int)(a.T - t0 < C ? a.T - t0 : C);
    __syncthreads();  // the previous chunk's tables and outputs are consumed
    stage();
    __syncthreads();
    if (c + 1 < a.nch) fetch(c + 1);  // in flight during this chunk
    // P_i = s . W_i and Qs_r = s . q_r, reduced over the row's 16 lanes; lane (r & 15)
    // keeps token r's pair in LDS (partial unrolling: fully unrolled, the scheduler hoists
    // every token's reads and runs out of registers)
#pragma unroll 4
    for (int r = 0; r < C; ++r) {
      const float4 w0 = *reinterpret_cast<const float4 *>(&sW[r][EL * lr]);
      const float4 w1 = *reinterpret_cast<const float4 *>(&sW[r][EL * lr + 4]);
      const float4 q0 = *reinterpret_cast<const float4 *>(&sQ[r][EL * lr]);
      const float4 q1 = *reinterpret_cast<const float4 *>(&sQ[r][EL * lr + 4]);
      float pw = s[0] * w0.x, pq = s[0] * q0.x;
      pw = __builtin_fmaf(s[1], w0.y, pw); pq = __builtin_fmaf(s[1], q0.y, pq);
      pw = __builtin_fmaf(s[2], w0.z, pw); pq = __builtin_fmaf(s[2], q0.z, pq);
      pw = __builtin_fmaf(s[3], w0.w, pw); pq = __builtin_fmaf(s[3], q0.w, pq);
      pw = __builtin_fmaf(s[4], w1.x, pw); pq = __builtin_fmaf(s[4], q1.x, pq);
      pw = __builtin_fmaf(s[5], w1.y, pw); pq = __builtin_fmaf(s[5], q1.y, pq);
      pw = __builtin_fmaf(s[6], w1.z, pw); pq = __builtin_fmaf(s[6], q1.z, pq);
      pw = __builtin_fmaf(s[7], w1.w, pw); pq = __builtin_fmaf(s[7], q1.w, pq);
      pw = group_sum_dpp<16>(pw);
      pq = group_sum_dpp<16>(pq);
      if (lr == (r & 15)) {
        sP[rl][r] = pw;
        sQs[rl][r] = pq;
      }
    }
    wave_lds_sync();  // each row's P and Qs come from its own wave
    // outputs: lane lr takes tokens lr and lr + 16 of this row
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 16 * h;
      float acc1 = 0.f, acc2 = 0.f;
#pragma unroll 2
      for (int i = 0; i < C; i += 4) {
        const float4 a1 = *reinterpret_cast<const float4 *>(&sA1[r][i]);
        const float4 a2 = *reinterpret_cast<const float4 *>(&sA2[r][i]);
        const float4 pp = *reinterpret_cast<const float4 *>(&sP[rl][i]);
        const float4 uu = *reinterpret_cast<const float4 *>(&sU[rl][i]);
        acc1 = __builtin_fmaf(a1.x, pp.x, acc1); acc2 = __builtin_fmaf(a2.x, uu.x, acc2);
        acc1 = __builtin_fmaf(a1.y, pp.y, acc1); acc2 = __builtin_fmaf(a2.y, uu.y, acc2);
        acc1 = __builtin_fmaf(a1.z, pp.z, acc1); acc2 = __builtin_fmaf(a2.z, uu.z, acc2);
        acc1 = __builtin_fmaf(a1.w, pp.w, acc1); acc2 = __builtin_fmaf(a2.w, uu.w, acc2);
      }
      sO[r][rl] = f32_to_bf16(__builtin_fmaf(sGm[r], sQs[rl][r] - acc1, acc2));
    }
    // state: s <- gam_31 s + sum_i (e_i U_i - gam_31 P_i) k_i
    const float gl = sGm[C - 1];
#pragma unroll
    for (int e = 0; e < EL; ++e) s[e] *= gl;
    auto upd = [&](float ci, int i) {
      const float4 k0 = *reinterpret_cast<const float4 *>(&sK[i][EL * lr]);
      const float4 k1 = *reinterpret_cast<const float4 *>(&sK[i][EL * lr + 4]);
      s[0] = __builtin_fmaf(ci, k0.x, s[0]); s[1] = __builtin_fmaf(ci, k0.y, s[1]);
      s[2] = __builtin_fmaf(ci, k0.z, s[2]); s[3] = __builtin_fmaf(ci, k0.w, s[3]);
      s[4] = __builtin_fmaf(ci, k1.x, s[4]); s[5] = __builtin_fmaf(ci, k1.y, s[5]);
      s[6] = __builtin_fmaf(ci, k1.z, s[6]); s[7] = __builtin_fmaf(ci, k1.w, s[7]);
    };
#pragma unroll 2
    for (int i = 0; i < C; i += 4) {
      const float4 pp = *reinterpret_cast<const float4 *>(&sP[rl][i]);
      const float4 uu = *reinterpret_cast<const float4 *>(&sU[rl][i]);
      const float4 ee = *reinterpret_cast<const float4 *>(&sE[i]);
      upd(__builtin_fmaf(ee.x, uu.x, -gl * pp.x), i);
      upd(__builtin_fmaf(ee.y, uu.y, -gl * pp.y), i + 1);
      upd(__builtin_fmaf(ee.z, uu.z, -gl * pp.z), i + 2);
      upd(__builtin_fmaf(ee.w, uu.w, -gl * pp.w), i + 3);
    }
    __syncthreads();
    if (tid < 2 * n) {
      const int r = tid >> 1, h = tid & 1;
      *reinterpret_cast<uint4 *>(a.out + ((size_t)(t0 + r) * a.n_v + j) * D + i0 + 8 * h) =
          *reinterpret_cast<const uint4 *>(&sO[r][8 * h]);
    }
  }
  *reinterpret_cast<float4 *>(srow) = float4{s[0], s[1], s[2], s[3]};
  *reinterpret_cast<float4 *>(srow + 4) = float4{s[4], s[5], s[6], s[7]};
}

hipError_t launch_gdn_chunked(const GdnArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_gdn_prep", k_gdn_prep, dim3((unsigned)a.n_v, (unsigned)a.nch), dim3(256), 0, s,
             a);
  MOE_LAUNCH("k_gdn_chunks", k_gdn_chunks, dim3((unsigned)a.n_v, kGdnD / 16), dim3(256), 0, s,
             a);
  return hipSuccess;
}

bool gdn_supported(int n_k, int n_v, int d_k, int d_v) {
  return n_k > 0 && n_v > 0 && n_v % n_k == 0 && d_k == kGdnD && d_v == kGdnD;
}

hipError_t launch_gdn_scan(const GdnArgs &a, hipStream_t s) {
  constexpr int RW = 4 * (64 / kGdnLanes);
  MOE_LAUNCH("k_gdn_scan", k_gdn_scan<kGdnLanes>, dim3((unsigned)a.n_v, kGdnD / RW), dim3(256), 0,
             s, a);
  return hipSuccess;
}

}  // namespace moe
