// gemm_grouped.hip -- grouped expert GEMMs of the prefill path on the MFMA units.
//
// "Optimizing On-Device Inference for Apple Silicon", section "Dequantize weights
// during matrix multiplication": the int4 weights are reconstructed one small tile at a
// time on chip and multiplied with the routed activation rows with fp32 accumulation;
// the expanded weight array never exists in device memory. Section "Match tile size to
// expert load": each expert's output is split into fixed-size tiles listed by the
// routing block map.
//
// Differences from the page's design, made for gfx950:
//   - Operands are fp16, not bf16: fp16 MFMA runs at the bf16 rate and keeps 3 more
//     mantissa bits of every reconstructed weight and of h; x (bf16) is exact in fp16.
//     Operands must stay inside the fp16 range (|value| < 65504).
//   - The reconstructed weights never touch LDS: each wave owns 64 weight rows and
//     dequantises their codes straight into MFMA B-operand registers (16 bytes of codes
//     per lane per K step). Only the gathered activation rows (shared by the four waves)
//     and the raw codes are staged in LDS.
//
// Tile: 128 slot rows x 256 weight rows, K in steps of 64 (one quantisation group).
// Wave w computes all 128 rows x weight rows {w's 64}: 4 x 2 tiles of
// v_mfma_f32_32x32x16_f16 (128 fp32 accumulators).
//   gate/up: weight rows = gate rows i0 + 32w .. +32 and the matching up rows, so the gate
//            and up accumulators of a (row, i) sit in the same lane and SwiGLU is applied
//            in registers; h is written in slot order [slots, I] fp16.
//   down:    weight rows = output columns n0 + 64w .. +64. A routed slot's row is scaled
//            by its routing weight and written fp16 in slot order; the shared expert's
//            rows are written fp32 in token order (section "Reduce intermediate and state
//            traffic": the output projection is combined with the routing score).
// MFMA K order: lane (n, half) of a B operand holds the 8 K of substep kk at
// 32*half + 8*kk (inside that chunk in the order 0,4,1,5,2,6,3,7 in which the packed
// dequantisation produces them), so over the 4 substeps a lane covers 32 consecutive K =
// 16 code bytes. The fp16 activation rows (x and h) are stored with the same order inside
// every 8-element chunk, so the A operand is a plain 16-byte LDS read.
// Pipeline: activation rows, codes, scales and biases travel global -> LDS directly
// (global_load_lds, no registers) into a 3-stage ring, issued two K steps ahead of use;
// each wave reads back its own codes and dequantises them one MFMA substep ahead.
// Scale and bias arrays must be 4-byte aligned and K must be a multiple of 128.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int BM = kTileM, BNW = 256, BK = 64;
constexpr int kStages = 3;                         // LDS ring depth (loads run 2 steps ahead)
constexpr int kABytes = BM * BK * 2;               // activation rows of one step: 16 KB
constexpr int kBBytes = 4 * 2 * 1024;              // codes: 4 waves x 2 columns x 64 lanes x 16 B
constexpr int kStageBytes = kABytes + kBBytes;
// Scales and biases travel as dwords: the dword at an even group index g holds groups g and
// g+1, i.e. K steps g and g+1, so they are loaded every other step into a 2-slot ring
// (4 arrays x 64 lanes x 4 B per wave and slot).
constexpr int kSSlot = 4 * 4 * 256;
constexpr int kSmemBytes = kStages * kStageBytes + 2 * kSSlot;  // 80 KB: two workgroups per CU
}  // namespace

MOE_DEV f16x2_t f16_pair_from_bf16(uint16_t v) {
  const _Float16 h = (_Float16)bf16_to_f32(v);
  return f16x2_t{h, h};
}

template <bool kGateUp>
__global__ __launch_bounds__(256, 2) void k_grouped(GroupedArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];

  // XCD-aware tile order: workgroup ids are dealt round-robin over the 8 XCDs; this map
  // gives each XCD all N tiles of one M tile back to back, so the activation rows of a
  // tile are fetched into that XCD's L2 once.
  const int nN = kGateUp ? a.I / (BNW / 2) : a.H / BNW;
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

  // Activation rows of one step land in LDS swizzled: 16-byte chunk c of row r sits at
  // chunk c ^ ((r >> 1) & 7) of the row, which keeps the MFMA operand reads (16 rows, one
  // chunk) free of bank conflicts. Each wave loads rows 32*wave .. +32 with 4 direct
  // loads of 8 rows; lane l fills physical chunk l % 8 of row l / 8 of such a group.
  const uint16_t *asrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 32 * wave + 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int rr = min(r, nvalid - 1);
    const uint16_t *row;
    if (kGateUp) {
      const int tok = (e == a.E) ? (row0 + rr) : a.sorted_tok[slot0 + rr];
      row = a.x16 + (size_t)tok * a.H;
    } else {
      row = a.h16 + (size_t)(slot0 + rr) * a.I;
    }
    asrc[q] = row + 8 * c;
  }

  // this lane's two B columns (weight rows) and K half
  const int bn = lane & 31, bh = lane >> 5;
  int wrow0, wrow1;
  if (kGateUp) {
    wrow0 = n_tile * (BNW / 2) + 32 * wave + bn;
    wrow1 = a.I + wrow0;
  } else {
    wrow0 = n_tile * BNW + 64 * wave + bn;
    wrow1 = wrow0 + 32;
  }
  const uint8_t *q_base = kGateUp ? a.wt.w13_q : a.wt.w2_q;
  const uint16_t *s_base = kGateUp ? a.wt.w13_s : a.wt.w2_s;
  const uint16_t *b_base = kGateUp ? a.wt.w13_b : a.wt.w2_b;
  const size_t r0 = (size_t)e * Nw + wrow0, r1 = (size_t)e * Nw + wrow1;
  const uint8_t *bq0 = q_base + r0 * (size_t)(K / 2) + 16 * bh;
  const uint8_t *bq1 = q_base + r1 * (size_t)(K / 2) + 16 * bh;
  const uint16_t *bs0 = s_base + r0 * (size_t)(K / kGroup), *bb0 = b_base + r0 * (size_t)(K / kGroup);
  const uint16_t *bs1 = s_base + r1 * (size_t)(K / kGroup), *bb1 = b_base + r1 * (size_t)(K / kGroup);

  // The direct-to-LDS loads and the step barrier are issued as inline assembly: the
  // compiler cannot tell the ring stages apart and would wait for every load in flight
  // (vmcnt(0)) before each LDS read and at each barrier, which serialises the pipeline.
  // Completion is tracked explicitly instead: before reading stage `st`, each wave waits
  // until only the loads of step st+1 are outstanding (6, plus 4 scale/bias dwords when
  // st+1 is even), then all waves meet at s_barrier. Compiler-generated vmcnt waits stay
  // correct (outstanding loads only add).
  // M0 holds the wave-uniform LDS byte address; lane l's data lands at M0 + l * size.
  // The s_nop covers the wait states a load that reads M0 needs after M0 is written.
  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
#define MOE_DMA16(gptr, lds)                                                            \
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %0, off"         \
               :: "v"(gptr), "s"(lds) : "memory", "m0")
#define MOE_DMA4(gptr, lds)                                                             \
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 1\n\tglobal_load_lds_dword %0, off"           \
               :: "v"(gptr), "s"(lds) : "memory", "m0")
  // issue the direct-to-LDS loads of K step `step` (6 memory instructions per wave, 10 on
  // even steps, which also fetch the scales and biases of this step and the next)
#define MOE_ISSUE(step)                                                                 \
  do {                                                                                  \
    const uint32_t base_ = smem_lds + ((step) % kStages) * kStageBytes;                 \
    const int k0_ = (step) * BK;                                                        \
    _Pragma("unroll") for (int q = 0; q < 4; ++q)                                       \
      MOE_DMA16(asrc[q] + k0_, base_ + (32 * wave_u + 8 * q) * 128);                    \
    const uint32_t bb_ = base_ + kABytes + wave_u * 2048;                               \
    MOE_DMA16(bq0 + k0_ / 2, bb_);                                                      \
    MOE_DMA16(bq1 + k0_ / 2, bb_ + 1024);                                               \
    if (((step) & 1) == 0) {                                                            \
      const uint32_t sb_ =                                                              \
          smem_lds + kStages * kStageBytes + (((step) >> 1) & 1) * kSSlot + wave_u * 1024; \
      MOE_DMA4(bs0 + (step), sb_);                                                      \
      MOE_DMA4(bb0 + (step), sb_ + 256);                                                \
      MOE_DMA4(bs1 + (step), sb_ + 512);                                                \
      MOE_DMA4(bb1 + (step), sb_ + 768);                                                \
    }                                                                                   \
  } while (0)

  f32x16_t acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m][0] = acc[m][1] = f32x16_t{};

  const int nsteps = K / BK;
  const int arow_l = lane & 31, ahalf = lane >> 5;
  // every lane's source pointers are computed (their loads done) before the first DMA
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  MOE_ISSUE(0);
  if (nsteps > 1) MOE_ISSUE(1);
  for (int st = 0; st < nsteps; ++st) {
    // this wave's loads of step st have landed (step st+1's may still be in flight),
    // then everyone's have, and everyone is done with the stage step st+2 will reuse
    if (st + 1 < nsteps) {
      if (st & 1)
        asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    } else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    if (st + 2 < nsteps) MOE_ISSUE(st + 2);
    const uint8_t *base = smem + (st % kStages) * kStageBytes;
    const uint8_t *bsrc = base + kABytes + wave * 2048;
    const uint32_t *sv = reinterpret_cast<const uint32_t *>(
        smem + kStages * kStageBytes + ((st >> 1) & 1) * kSSlot + wave * 1024);
    const uint4 q0 = *reinterpret_cast<const uint4 *>(bsrc + 16 * lane);
    const uint4 q1 = *reinterpret_cast<const uint4 *>(bsrc + 1024 + 16 * lane);
    const int sh = 16 * (st & 1);
    const f16x2_t s0 = f16_pair_from_bf16((uint16_t)(sv[lane] >> sh));
    const f16x2_t b0 = f16_pair_from_bf16((uint16_t)(sv[64 + lane] >> sh));
    const f16x2_t s1 = f16_pair_from_bf16((uint16_t)(sv[128 + lane] >> sh));
    const f16x2_t b1 = f16_pair_from_bf16((uint16_t)(sv[192 + lane] >> sh));
    const uint32_t w0[4] = {q0.x, q0.y, q0.z, q0.w}, w1[4] = {q1.x, q1.y, q1.z, q1.w};
    f16x8_t bc0 = __builtin_bit_cast(f16x8_t, dequant8_pk(w0[0], s0, b0));
    f16x8_t bc1 = __builtin_bit_cast(f16x8_t, dequant8_pk(w1[0], s1, b1));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f16x8_t av[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 32 * m + arow_l;
        const int pc = (4 * ahalf + kk) ^ ((r >> 1) & 7);
        av[m] = *reinterpret_cast<const f16x8_t *>(base + r * 128 + pc * 16);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[m], bc0, acc[m][0], 0, 0, 0);
        acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[m], bc1, acc[m][1], 0, 0, 0);
      }
      if (kk < 3) {
        // next substep's weights while the MFMAs above run
        bc0 = __builtin_bit_cast(f16x8_t, dequant8_pk(w0[kk + 1], s0, b0));
        bc1 = __builtin_bit_cast(f16x8_t, dequant8_pk(w1[kk + 1], s1, b1));
      }
    }
  }
#undef MOE_ISSUE
#undef MOE_DMA16
#undef MOE_DMA4

  // 32x32 accumulator layout: lane l holds column l%32, register r holds row
  // 8*(r/4) + 4*(l/32) + r%4.
  const int col = lane & 31, rq4 = (lane >> 5) * 4;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * m + (r >> 2) * 8 + rq4 + (r & 3);
      if (row >= nvalid) continue;
      const size_t slot = (size_t)(slot0 + row);
      if (kGateUp) {
        // h keeps the chunk order of the fp16 operand rows (it is the down GEMM's A)
        const int i = n_tile * (BNW / 2) + 32 * wave + col;
        a.h16[slot * a.I + (i & ~7) + kChunkPos[i & 7]] =
            f32_to_f16(silu(acc[m][0][r]) * acc[m][1][r]);
      } else {
        const int n = n_tile * BNW + 64 * wave + col;
        if (e < a.E) {
          const float wv = a.slot_w[slot];
          a.out[slot * a.H + n] = f32_to_f16(wv * acc[m][0][r]);
          a.out[slot * a.H + n + 32] = f32_to_f16(wv * acc[m][1][r]);
        } else {
          const size_t t = (size_t)(row0 + row);
          a.out_sh[t * a.H + n] = acc[m][0][r];
          a.out_sh[t * a.H + n + 32] = acc[m][1][r];
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
  MOE_LAUNCH("k_grouped_gateup", (k_grouped<true>),
             dim3(grouped_grid(a.max_tiles, a.I / (BNW / 2))), dim3(256), 0, s, a);
  return hipSuccess;
}

hipError_t launch_grouped_down(const GroupedArgs &a, hipStream_t s) {
  MOE_LAUNCH("k_grouped_down", (k_grouped<false>), dim3(grouped_grid(a.max_tiles, a.H / BNW)),
             dim3(256), 0, s, a);
  return hipSuccess;
}

}  // namespace moe
