// gemm_grouped.hip -- grouped expert GEMMs of the prefill path on the MFMA units.
//
// "Optimizing On-Device Inference for Apple Silicon", section "Dequantize weights
// during matrix multiplication": the int4 weights are reconstructed one small tile at a
// time in on-chip memory (LDS here) and multiplied with the routed activation rows with
// fp32 accumulation; the expanded weight array never exists in device memory. Section
// "Match tile size to expert load": each expert's output is split into fixed-size tiles
// listed by the routing block map.
//
// Operand precision differs from the page (which reconstructs bf16 for a bf16 matrix
// unit): gfx950 runs fp16 MFMA at the bf16 rate, and fp16 keeps 3 more mantissa bits of
// every reconstructed weight and of h. x (bf16) is exact in fp16. Operands must stay
// inside the fp16 range (|value| < 65504).
//
// Tile: 128 slot rows x 128 weight rows, K in steps of 64 (one quantisation group).
// 4 waves in a 2x2 layout, each computing 64x64 with v_mfma_f32_32x32x16_f16.
//   gate/up: the 128 weight rows are 64 gate rows i0.. and the 64 matching up rows, so a
//            wave holds gate and up accumulators of the same (row, i) and applies
//            SwiGLU in registers; h is written in slot order [slots, I] fp16.
//   down:    128 output columns of W2. A routed slot's row is scaled by its routing
//            weight and written fp16 in slot order; the shared expert's rows are written
//            fp32 in token order (section "Reduce intermediate and state traffic": the
//            output projection is combined with the routing score).
// Operand staging: LDS double buffer; global loads of step s+1 are issued before the
// MFMAs of step s, dequantised and stored after them.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int BM = kTileM, BN = 128, BK = 64;
constexpr int LDP = BK + 8;  // LDS row pitch in fp16 elements (16-byte pad)
}  // namespace

template <bool kGateUp>
__global__ __launch_bounds__(256) void k_grouped(GroupedArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDP];

  // XCD-aware tile order: workgroup ids are dealt round-robin over the 8 XCDs, so the
  // id -> tile map gives each XCD all N tiles of one M tile back to back (the
  // activation rows of a tile are then reused from that XCD's L2).
  const int nN = kGateUp ? a.I / 64 : a.H / BN;
  const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
  const int n_tile = j % nN, m_tile = (j / nN) * 8 + xcd;
  if (m_tile >= *a.n_tiles) return;
  const int2 tile = a.tiles[m_tile];
  const int e = tile.x, row0 = tile.y;
  const int gbase = a.offsets[e];
  const int nvalid = min(BM, a.offsets[e + 1] - gbase - row0);
  const int slot0 = gbase + row0;
  const int K = kGateUp ? a.H : a.I;
  const int Nw = kGateUp ? 2 * a.I : a.H;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> LDS assignment: row lr, half lh (32 elements = 64 B of A, 16 B of codes)
  const int lr = tid >> 1, lh = tid & 1;
  const int rr = min(lr, nvalid - 1);
  const uint16_t *arow;
  if (kGateUp) {
    const int tok = (e == a.E) ? (row0 + rr) : a.sorted_tok[slot0 + rr];
    arow = a.x16 + (size_t)tok * a.H;
  } else {
    arow = a.h16 + (size_t)(slot0 + rr) * a.I;
  }
  int wrow;
  if (kGateUp)
    wrow = lr < 64 ? n_tile * 64 + lr : a.I + n_tile * 64 + (lr - 64);
  else
    wrow = n_tile * BN + lr;
  const size_t wr = (size_t)e * Nw + wrow;
  const uint8_t *bq = (kGateUp ? a.wt.w13_q : a.wt.w2_q) + wr * (size_t)(K / 2);
  const uint16_t *bs = (kGateUp ? a.wt.w13_s : a.wt.w2_s) + wr * (size_t)(K / kGroup);
  const uint16_t *bb = (kGateUp ? a.wt.w13_b : a.wt.w2_b) + wr * (size_t)(K / kGroup);

  uint4 ra0, ra1, ra2, ra3, rq;
  uint16_t rs, rb;
  auto gload = [&](int k0) {
    const uint4 *p = reinterpret_cast<const uint4 *>(arow + k0 + lh * 32);
    ra0 = p[0];
    ra1 = p[1];
    ra2 = p[2];
    ra3 = p[3];
    rq = *reinterpret_cast<const uint4 *>(bq + k0 / 2 + lh * 16);
    rs = bs[k0 / kGroup];
    rb = bb[k0 / kGroup];
  };
  auto lstore = [&](int buf) {
    uint4 *pa = reinterpret_cast<uint4 *>(&As[buf][lr * LDP + lh * 32]);
    pa[0] = ra0;
    pa[1] = ra1;
    pa[2] = ra2;
    pa[3] = ra3;
    const float s = bf16_to_f32(rs), b = bf16_to_f32(rb);
    uint4 *pb = reinterpret_cast<uint4 *>(&Bs[buf][lr * LDP + lh * 32]);
    pb[0] = dequant8_f16(rq.x, s, b);
    pb[1] = dequant8_f16(rq.y, s, b);
    pb[2] = dequant8_f16(rq.z, s, b);
    pb[3] = dequant8_f16(rq.w, s, b);
  };

  // B sub-tile rows of this wave
  const int nb0 = kGateUp ? 32 * wn : 64 * wn;
  const int nb1 = kGateUp ? 64 + 32 * wn : 64 * wn + 32;
  const int frow = lane & 31, fk = (lane >> 5) * 8;

  f32x16_t acc00 = {}, acc01 = {}, acc10 = {}, acc11 = {};
  const int nsteps = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int cur = st & 1;
    if (st + 1 < nsteps) gload((st + 1) * BK);
    const uint16_t *A_ = As[cur];
    const uint16_t *B_ = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ko = kk * 16 + fk;
      const f16x8_t a0 = *reinterpret_cast<const f16x8_t *>(A_ + (wm * 64 + frow) * LDP + ko);
      const f16x8_t a1 =
          *reinterpret_cast<const f16x8_t *>(A_ + (wm * 64 + 32 + frow) * LDP + ko);
      const f16x8_t b0 = *reinterpret_cast<const f16x8_t *>(B_ + (nb0 + frow) * LDP + ko);
      const f16x8_t b1 = *reinterpret_cast<const f16x8_t *>(B_ + (nb1 + frow) * LDP + ko);
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc00, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, acc01, 0, 0, 0);
      acc10 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, acc10, 0, 0, 0);
      acc11 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc11, 0, 0, 0);
    }
    if (st + 1 < nsteps) lstore(cur ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane l holds column l%32, register r holds row
  // 8*(r/4) + 4*(l/32) + r%4.
  const int col = lane & 31, rq4 = (lane >> 5) * 4;
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const f32x16_t &c0 = ms ? acc10 : acc00;
    const f32x16_t &c1 = ms ? acc11 : acc01;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm * 64 + ms * 32 + (r >> 2) * 8 + rq4 + (r & 3);
      if (m >= nvalid) continue;
      const size_t slot = (size_t)(slot0 + m);
      if (kGateUp) {
        const int i = n_tile * 64 + wn * 32 + col;
        a.h16[slot * a.I + i] = f32_to_f16(silu(c0[r]) * c1[r]);
      } else {
        const int n = n_tile * BN + wn * 64 + col;
        if (e < a.E) {
          const float wv = a.slot_w[slot];
          a.out[slot * a.H + n] = f32_to_f16(wv * c0[r]);
          a.out[slot * a.H + n + 32] = f32_to_f16(wv * c1[r]);
        } else {
          const size_t t = (size_t)(row0 + m);
          a.out_sh[t * a.H + n] = c0[r];
          a.out_sh[t * a.H + n + 32] = c1[r];
        }
      }
    }
  }
}

static unsigned grouped_grid(int max_tiles, int nN) {
  const int mt_pad = (max_tiles + 7) / 8 * 8;
  return (unsigned)(mt_pad * nN);
}

hipError_t launch_grouped_gateup(const GroupedArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_grouped_gateup", (k_grouped<true>), dim3(grouped_grid(a.max_tiles, a.I / 64)),
             dim3(256), 0, s, a);
  return hipSuccess;
}

hipError_t launch_grouped_down(const GroupedArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_grouped_down", (k_grouped<false>), dim3(grouped_grid(a.max_tiles, a.H / BN)),
             dim3(256), 0, s, a);
  return hipSuccess;
}

}  // namespace moe
