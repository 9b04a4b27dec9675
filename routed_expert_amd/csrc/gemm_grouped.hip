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
// Tile: up to 128 slot rows (160 when a group's short remainder joins its last full tile)
// x 256 weight rows, K in steps of 64 (one quantisation group). Wave w computes all rows x
// weight rows {w's 64}: MB x 2 tiles of v_mfma_f32_32x32x16_f16 (up to 160 fp32
// accumulators), MB = the tile's 32-row blocks that hold valid rows.
//   gate/up: weight rows = gate rows i0 + 32w .. +32 and the matching up rows, so the gate
//            and up accumulators of a (row, i) sit in the same lane and SwiGLU is applied
//            in registers; h is written in slot order [slots, I] fp16.
//   down:    weight rows = output columns n0 + 64w .. +64. Every routed row is written
//            fp16 in slot order, scaled by its routing weight (section "Reduce intermediate
//            and state traffic": the output projection is combined with the routing
//            score). The shared expert's down projection runs over token tiles with the
//            weighted combine in its epilogue (k_shared_down_combine).
// MFMA K order: lane (n, half) of a B operand holds the 8 K of substep kk at
// 32*half + 8*kk (inside that chunk in the order 0,4,1,5,2,6,3,7 in which the packed
// dequantisation produces them), so over the 4 substeps a lane covers 32 consecutive K =
// 16 code bytes. The fp16 activation rows (x and h) are stored with the same order inside
// every 8-element chunk, so the A operand is a plain 16-byte LDS read.
// Pipeline: activation rows, codes, scales and biases travel global -> LDS directly
// (global_load_lds, no registers) into a 3-stage ring, issued two K steps ahead of use;
// each wave reads back its own codes and dequantises them one MFMA substep ahead, between
// the MFMAs of the substep before (the matrix unit runs an MFMA while the wave issues
// independent vector instructions, so about six of them per MFMA cost no time).
// Scale and bias arrays must be 4-byte aligned and K must be a multiple of 128.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int BM = kTileM, BNW = 256, BK = 64;
constexpr int kStages = 3;                         // LDS ring depth (loads run 2 steps ahead)
constexpr int kABytes = BM * BK * 2;               // activation rows of one step: 16 KB
constexpr int kBBytes = 4 * 2 * 1024;              // codes: 4 waves x 2 columns x 64 lanes x 16 B
// Scales and biases of one step (one K group): 4 waves x 64 weight rows x {scale, bias}.
constexpr int kSBBytes = 4 * 256;
constexpr int kSmemBytes = 80 * 1024;              // two workgroups per CU
// LDS word of the persistent launch's next ticket, above everything a tile uses
constexpr int kTicketOff = kSmemBytes - 16;
// Routing weights of a down tile's rows (up to 160 floats), requested at the tile's start into
// LDS above the ring and below the ticket word, read by the epilogue
constexpr int kSwOff = kTicketOff - 5 * 32 * 4;
// A tile of five 32-row blocks (an expert's last full tile with its short remainder, see
// group_tables) has 20 KB of activation rows per step; three such stages would not fit two
// workgroups per CU, so it runs a two-stage ring (loads one K step ahead instead of two).
constexpr int kMaxMB = 5;
template <int MB> constexpr int ring_stages() { return MB > 4 ? 2 : kStages; }
template <int MB> constexpr int a_stage_bytes() { return (MB > 4 ? MB : 4) * 32 * BK * 2; }
// Expanded-weight variant (separate dequantisation pass, an ablation): each wave's B operand
// of a step is 8 KB of fp16 instead of 2 KB of codes, so a stage is 48 KB and the 144 KB
// ring leaves room for one workgroup per CU.
constexpr int kXBBytes = 4 * 8 * 1024;
constexpr int kXSmemBytes = kStages * (kABytes + kXBBytes);
}  // namespace

MOE_DEV f16x2_t f16_pair_from_bf16(uint16_t v) {
  const _Float16 h = (_Float16)bf16_to_f32(v);
  return f16x2_t{h, h};
}

template <int N>
MOE_DEV void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One tile: rows [row0, row0 + nvalid) of group e, weight rows of N tile n_tile. MB is the
// number of 32-row blocks holding valid rows (1..4, or 5 for a full tile that took in its
// group's short remainder); blocks past them are neither loaded nor multiplied, so a
// group's last, partial tile costs MFMA work in proportion to its rows.
// kX: B operands come ready-made from the expanded fp16 weights (launch_expand) instead of
// being dequantised from the codes; every other step is the same, and so are the results.
// kComb (down projection of the shared expert over token tiles only): instead of storing the
// tile, the epilogue adds each token's k routed outputs (already weighted) in a fixed order and
// the residual, and writes y in bf16 (the weighted combine, fused).
template <bool kGateUp, int MB, bool kX, bool kComb = false>
MOE_DEV void grouped_tile(const GroupedArgs &a, uint8_t *smem, int e, int row0, int nvalid,
                          int n_tile, int wave, int32_t *tk = nullptr) {
  constexpr int kSt = ring_stages<MB>();                 // ring depth
  constexpr int kAB = a_stage_bytes<MB>();               // activation rows of one stage
  constexpr int kBB = kX ? kXBBytes : kBBytes;          // weight operands of one stage
  constexpr int kSB = kAB + kBB + (kX ? 0 : kSBBytes);   // bytes of one ring stage
  constexpr int kLB = kX ? 8 : 3;  // B loads per wave and step (codes 2 + scales 1)
  static_assert(kSt * kSB <= (kX ? kXSmemBytes : kTicketOff), "ring does not fit the LDS");
  // Down tiles multiply with the operands exchanged (weights first): the product is the
  // transposed tile, so a lane's accumulators hold four adjacent output columns of one row,
  // which go to LDS in one write instead of four. The operand fragments of the two forms
  // have the same register layout, and every sum is the same.
  constexpr bool kWT = !kGateUp;
  // tables are uniform per tile; in the persistent launch the compiler cannot prove it (the
  // loads follow stores of earlier items), so the values are made scalar explicitly
  const int gbase = __builtin_amdgcn_readfirstlane(a.offsets[e]);
  const int slot0 = gbase + row0;
  const int K = kGateUp ? a.H : a.I;
  // wave (uniform) comes from the caller; the lane index is formed here by an opaque
  // instruction pair. In the persistent launch the tile runs in a loop, and the lane-dependent
  // offsets would otherwise be computed once before it and held in registers across it
  // (spilled, at 256 in use), as would the thread index register itself.
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int tid = 64 * wave + lane;

  // Activation rows of one step land in LDS swizzled: 16-byte chunk c of row r sits at
  // chunk c ^ ((r >> 1) & 7) of the row, which keeps the MFMA operand reads (16 rows, one
  // chunk) free of bank conflicts. The 4*MB groups of 8 rows are spread over the waves:
  // direct load j of wave w fills row group w + 4j; lane l fills physical chunk l % 8 of
  // row l / 8 of its group.
  // Every direct load takes a wave-uniform 64-bit base in SGPRs and a 32-bit byte offset per
  // lane (the instruction's saddr form): the activation rows' base is x16 (gathered tokens;
  // T * H * 2 < 2^32 bytes, which the host guarantees by splitting larger calls) or the
  // tile's first h row, the weights' base is the wave's block, and one lane offset (16 l)
  // serves codes, scales and expanded weights.
  const uint8_t *abase = kGateUp ? reinterpret_cast<const uint8_t *>(a.x16)
                                 : reinterpret_cast<const uint8_t *>(a.h16 + (size_t)slot0 * a.I);
  uint32_t aoff[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int r = 8 * (wave + 4 * j) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int rr = min(r, nvalid - 1);
    if (kGateUp) {
      const int tok = (e == a.E) ? (row0 + rr) : a.sorted_tok[slot0 + rr];
      aoff[j] = (uint32_t)tok * (uint32_t)(2 * a.H) + 16u * c;
    } else {
      aoff[j] = (uint32_t)rr * (uint32_t)(2 * a.I) + 16u * c;
    }
  }
  const uint32_t loff = 16u * lane;

  // This wave's weight rows are one 64-row block of the tiled layout: gate rows 32w..+32
  // of the N tile and the matching up rows (gate/up), or output rows 64w..+64 (down). Per
  // K step the block's codes are 2 KB contiguous (column block c = rows 32c..32c+31 at
  // c * 1 KB); its scales and biases are tiled 1 KB per four steps, lane l = 32c + row
  // holding 4 steps x {scale, bias} in 16 bytes, of which each step loads its 4 bytes.
  const int wave_u = wave;
  const int nb = kGateUp ? 2 * a.I / 64 : a.H / 64;
  const int blk = n_tile * 4 + wave_u;
  const int ns = K / BK, ns4 = (ns + 3) / 4;
  const uint8_t *tq = (kGateUp ? a.wt.w13_t : a.wt.w2_t) + ((size_t)e * nb + blk) * ns * 2048;
  const uint8_t *tsb = reinterpret_cast<const uint8_t *>(
      (kGateUp ? a.wt.w13_tsb : a.wt.w2_tsb) + ((size_t)e * nb + blk) * ns4 * 512);
  // expanded weights: the same block's 8 KB of fp16 per K step, 1 KB per (column block,
  // substep), lane l's 8 values at 16 l
  const uint8_t *txq = kX ? reinterpret_cast<const uint8_t *>(kGateUp ? a.w13_x : a.w2_x) +
                                ((size_t)e * nb + blk) * ns * 8192
                          : nullptr;

  // The direct-to-LDS loads and the step barrier are issued as inline assembly: the
  // compiler cannot tell the ring stages apart and would wait for every load in flight
  // (vmcnt(0)) before each LDS read and at each barrier, which serialises the pipeline.
  // Completion is tracked explicitly instead: every step issues the same MB + kLB loads per
  // wave (past the last step, a harmless reload of the last step's sources into the free
  // stage), so during step st each wave waits until only the loads of step st+2 are
  // outstanding and its own loads of step st+1 have landed; the barrier at the top of step
  // st+1 then covers every wave's. Compiler-generated vmcnt waits stay correct (outstanding
  // loads only add). The step body has no branches: one scheduling region from the DMA
  // issue to the mid-step wait, in which the dequantisation interleaves with the MFMAs.
  // M0 holds the wave-uniform LDS byte address; lane l's data lands at M0 + l * size.
  // The s_nop covers the wait states a load that reads M0 needs after M0 is written. M0 is
  // listed as clobbered, and hipcc warns that it does not preserve a reserved register across
  // such a statement: nothing else in these kernels uses M0 (in the generated code every M0
  // write is one of these statements and only these loads read it).
  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
#define MOE_DMA16(voff, sbase, lds)                                                     \
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %0, %1"          \
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0")
#define MOE_DMA4(voff, sbase, lds)                                                      \
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 1\n\tglobal_load_lds_dword %0, %1"            \
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0")
  // issue the direct-to-LDS loads of K step `step` into ring stage `slot` (MB + 3 memory
  // instructions per wave: activation rows, two code blocks, the step's scales and biases;
  // expanded weights: MB + 8)
#define MOE_ISSUE(step, slot)                                                           \
  do {                                                                                  \
    const uint32_t base_ = smem_lds + (slot) * kSB;                                     \
    const uint8_t *as_ = abase + (size_t)(step) * (BK * 2);                             \
    _Pragma("unroll") for (int j = 0; j < MB; ++j)                                      \
      MOE_DMA16(aoff[j], as_, base_ + (wave_u + 4 * j) * 1024);                         \
    if constexpr (kX) {                                                                 \
      const uint32_t bb_ = base_ + kAB + wave_u * 8192;                                 \
      _Pragma("unroll") for (int q = 0; q < 8; ++q)                                     \
        MOE_DMA16(loff, txq + (size_t)(step) * 8192 + q * 1024, bb_ + q * 1024);        \
    } else {                                                                            \
      const uint32_t bb_ = base_ + kAB + wave_u * 2048;                                 \
      MOE_DMA16(loff, tq + (size_t)(step) * 2048, bb_);                                 \
      MOE_DMA16(loff, tq + (size_t)(step) * 2048 + 1024, bb_ + 1024);                   \
      MOE_DMA4(loff, tsb + (size_t)((step) >> 2) * 1024 + 4 * ((step) & 3),             \
               base_ + kAB + kBB + wave_u * 256);                                       \
    }                                                                                   \
  } while (0)

  f32x16_t acc[MB][2];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m][0] = acc[m][1] = f32x16_t{};

  const int nsteps = K / BK;
  // A operand of lane l: row 32m + l % 32, logical chunk 4*(l / 32) + kk of the step
  const int arow_l = lane & 31, ahalf = lane >> 5, asw = (arow_l >> 1) & 7;

  // This wave's codes, scales and biases of a step come from its own direct loads, so
  // they are read into registers during the third substep of the step before, once this
  // wave's loads of that step have landed, without a barrier; only the activation rows,
  // which all four waves load together, wait for the step barrier.
  uint32_t w0[4], w1[4];
  f16x2_t s0, b0, s1, b1, s0q, s1q;
  uint4 bx[8];  // expanded weights: the step's B operands, [column block][substep]
  const int bn = lane & 31, bh = lane >> 5;
#define MOE_READ_BX(slot)                                                               \
  do {                                                                                  \
    const uint8_t *bsrc_ = smem + (slot) * kSB + kAB + wave * 8192 + 16 * lane;         \
    _Pragma("unroll") for (int q = 0; q < 8; ++q)                                       \
      bx[q] = *reinterpret_cast<const uint4 *>(bsrc_ + q * 1024);                       \
  } while (0)
#define MOE_READ_B(slot)                                                                \
  do {                                                                                  \
    const uint8_t *bsrc_ = smem + (slot) * kSB + kAB + wave * 2048 + 32 * bn + 16 * bh; \
    const uint4 q0_ = *reinterpret_cast<const uint4 *>(bsrc_);                          \
    const uint4 q1_ = *reinterpret_cast<const uint4 *>(bsrc_ + 1024);                   \
    const uint32_t *sv_ = reinterpret_cast<const uint32_t *>(                           \
        smem + (slot) * kSB + kAB + kBB + wave * 256 + 4 * bn);                         \
    const uint32_t sb0_ = sv_[0], sb1_ = sv_[32];                                       \
    s0 = f16_pair_from_bf16((uint16_t)sb0_);                                            \
    b0 = f16_pair_from_bf16((uint16_t)(sb0_ >> 16));                                    \
    s1 = f16_pair_from_bf16((uint16_t)sb1_);                                            \
    b1 = f16_pair_from_bf16((uint16_t)(sb1_ >> 16));                                    \
    s0q = s0 * f16x2_t{(_Float16)0.0625f, (_Float16)0.0625f};                           \
    s1q = s1 * f16x2_t{(_Float16)0.0625f, (_Float16)0.0625f};                           \
    w0[0] = q0_.x; w0[1] = q0_.y; w0[2] = q0_.z; w0[3] = q0_.w;                         \
    w1[0] = q1_.x; w1[1] = q1_.y; w1[2] = q1_.z; w1[3] = q1_.w;                         \
  } while (0)

  // every lane's source pointers are computed (their loads done) before the first DMA
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // Down tiles of routed experts: the rows' routing weights travel to LDS with the first
  // step's operands (wave w fetches rows 64w .. 64w+63, past the tile's rows the last row's
  // weight again, which no stored row uses), so the epilogue does not wait for them. They are
  // older than every load of the ring, so the ring's first wait covers them.
  constexpr bool kPreSw = !kGateUp && !kComb && !kX;
  if constexpr (kPreSw) {
    static_assert(kSt * kSB <= kSwOff, "routing weights overlap the ring");
    if (e < a.E && 64 * wave < 32 * MB) {
      const uint32_t voff = 4u * (uint32_t)min(64 * wave + lane, nvalid - 1);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 1\n\tglobal_load_lds_dword %0, %1"
                   :: "v"(voff), "s"(a.slot_w + slot0), "s"(smem_lds + kSwOff + 256 * wave)
                   : "memory", "m0");
    }
  }
  // fused combine: the routed slots of this tile's tokens (row r, rank j at r * k + j),
  // requested now so that their latency hides behind the K loop
  int32_t slot_pre[2] = {0, 0};
  if constexpr (kComb) {
    static_assert(MB <= 2, "the fused combine takes token tiles of at most 64 rows");
#pragma unroll
    for (int q = 0; q < 2; ++q)
      slot_pre[q] = a.slot_of[(size_t)row0 * a.k + min(tid + 256 * q, nvalid * a.k - 1)];
  }
  MOE_ISSUE(0, 0);
  if constexpr (kSt > 2) {
    MOE_ISSUE(min(1, nsteps - 1), 1);
    wait_vmcnt<MB + kLB>();  // step 0's own loads: only stage 1's are younger
  } else {
    wait_vmcnt<0>();
  }
  // B operands of substep kk of the step whose codes (or expanded weights) are loaded
#define MOE_B_OPS(kk)                                                                   \
  do {                                                                                  \
    if constexpr (kX) {                                                                 \
      bc0 = __builtin_bit_cast(f16x8_t, bx[(kk)]);                                      \
      bc1 = __builtin_bit_cast(f16x8_t, bx[4 + (kk)]);                                  \
    } else {                                                                            \
      bc0 = __builtin_bit_cast(f16x8_t, dequant8_pk_q(w0[(kk)], s0, s0q, b0));          \
      bc1 = __builtin_bit_cast(f16x8_t, dequant8_pk_q(w1[(kk)], s1, s1q, b1));          \
    }                                                                                   \
  } while (0)
  f16x8_t bc0, bc1;
  if constexpr (kX)
    MOE_READ_BX(0);
  else
    MOE_READ_B(0);
  MOE_B_OPS(0);
  int slot = 0;  // ring stage of step st
  for (int st = 0; st < nsteps; ++st) {
    // every wave's loads of step st have landed (each wave waited for its own before its
    // mid-step read of step st's codes), and every wave is done with the stage that step
    // st + kSt - 1 will reuse
    asm volatile("s_barrier" ::: "memory");
    const int nslot = slot + 1 == kSt ? 0 : slot + 1;          // stage of step st + 1
    const int fslot = slot == 0 ? kSt - 1 : slot - 1;          // stage of step st + kSt - 1
    const uint8_t *arow = smem + slot * kSB + arow_l * 128;
    // A fragments are double-buffered: substep kk+1's are read while kk's MFMAs run
    f16x8_t av[2][MB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
      av[0][m] = *reinterpret_cast<const f16x8_t *>(arow + m * 4096 + ((4 * ahalf) ^ asw) * 16);
    MOE_ISSUE(min(st + kSt - 1, nsteps - 1), fslot);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
          av[(kk + 1) & 1][m] = *reinterpret_cast<const f16x8_t *>(
              arow + m * 4096 + ((4 * ahalf + kk + 1) ^ asw) * 16);
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if constexpr (kWT) {
          acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bc0, av[kk & 1][m], acc[m][0], 0, 0, 0);
          acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bc1, av[kk & 1][m], acc[m][1], 0, 0, 0);
        } else {
          acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[kk & 1][m], bc0, acc[m][0], 0, 0, 0);
          acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[kk & 1][m], bc1, acc[m][1], 0, 0, 0);
        }
      }
      // the next substep's weights while these MFMAs run
      if (kk < 3) MOE_B_OPS(kk + 1);
      if (kk == 2) {
        // the next step's codes, scales and biases (past the last step: the reloaded
        // stage, unused), once this wave's loads of step st+1 have landed, so that their
        // dequantisation overlaps the last substep's MFMAs
        wait_vmcnt<(kSt > 2 ? MB + kLB : 0)>();
        if constexpr (kX)
          MOE_READ_BX(nslot);
        else
          MOE_READ_B(nslot);
      }
      if (kk == 3) MOE_B_OPS(0);
      // A wave issues in order, and the matrix unit runs one MFMA while the same wave issues
      // independent vector instructions: spread the dequantisation and the LDS reads between
      // the MFMAs (a few VALU per MFMA) instead of leaving them in a block after the last one.
#pragma unroll
      for (int i = 0; i < 2 * MB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // up to 4 VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // up to 1 LDS read
      }
    }
    slot = nslot;
  }
  wait_vmcnt<0>();  // the reloads past the last step land before the stages are reused
#undef MOE_B_OPS
#undef MOE_READ_BX
#undef MOE_READ_B
#undef MOE_ISSUE
#undef MOE_DMA4
#undef MOE_DMA16

  // 32x32 accumulator layout: lane l holds column l%32, register r holds row
  // 8*(r/4) + 4*(l/32) + r%4. The tile leaves through LDS (the stages are free now): each
  // wave writes its fp16 results into a row-major tile, then every thread copies 16-byte
  // pieces of whole rows to global memory, instead of 2-byte stores scattered by the
  // accumulator layout. Rows are padded by 16 bytes, so the two rows an instruction
  // writes (l < 32 and l >= 32) fall into different bank halves.
  const int col = lane & 31, rq4 = (lane >> 5) * 4;
  __syncthreads();  // every wave is done reading the stages
  // persistent launch: the workgroup's next ticket, requested here (few registers live) and
  // stored to its LDS word once the tile is written, so its latency hides behind the epilogue
  int32_t tn = 0;
  if (tk && tid == 0) tn = __hip_atomic_fetch_add(tk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if constexpr (kGateUp) {
    // h: rows x 128 columns, stored in the chunk order of the fp16 operand rows (h is the
    // down GEMM's A operand)
    constexpr int HP = 128 + 8;
    _Float16 *ht = reinterpret_cast<_Float16 *>(smem);
    const int il = 32 * wave + col;
    const int pos = (il & ~7) + kChunkPos[il & 7];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * m + (r >> 2) * 8 + rq4 + (r & 3);
        ht[row * HP + pos] = (_Float16)(silu_fast(acc[m][0][r]) * acc[m][1][r]);
      }
    __syncthreads();
    // In the persistent launch a down tile may run on another XCD, whose L2 does not see
    // this one's: h is written through to memory (sc1), where that L2 fetches it.
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    for (int rr = tid >> 4; rr < nvalid; rr += 16) {
      uint16_t *dst = a.h16 + (size_t)(slot0 + rr) * a.I + n_tile * (BNW / 2) + 8 * (tid & 15);
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ht + rr * HP + 8 * (tid & 15));
      if (tk)
        asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"((uint64_t)(uintptr_t)dst),
                     "v"(v) : "memory");
      else
        *reinterpret_cast<u32x4_t *>(dst) = v;
    }
  } else if constexpr (kComb) {
    // y[t] = shared(x_t) + sum_j out[slot_of[t, j]] (+ residual[t]) over this tile's 256
    // columns, fp32 in that order, bf16 out. The shared result of every row goes through LDS
    // in fp32, the routed slots (requested before the K loop) beside it; then thread (row,
    // 8 columns) gathers the routed rows with 16-byte loads, four rows at a time with all
    // their loads in flight together (rows past the tile repeat its last row's loads and are
    // not stored, so no load sits under a branch), and writes 16 bytes of y per row.
    constexpr int SP = BNW + 4;
    float *st = reinterpret_cast<float *>(smem);
    int32_t *s_slot = reinterpret_cast<int32_t *>(smem + 32 * MB * SP * 4);
    static_assert(64 * SP * 4 + 64 * kMaxTopK * 4 <= kTicketOff, "combine staging");
    const int k = a.k;
    const int cc = 8 * (tid & 31), col0 = n_tile * BNW + cc;
    constexpr int kCombRows = 4;  // rows per thread gathered together
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (tid + 256 * q < 64 * kMaxTopK) s_slot[tid + 256 * q] = slot_pre[q];
    // transposed accumulators: lane l holds token row 32m + l%32, register r the column
    // 8*(r/4) + 4*(l/32) + r%4 of its 32-column block
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4 *>(st + (32 * m + col) * SP + 64 * wave + 32 * nb + 8 * g +
                                      rq4) =
              make_float4(acc[m][nb][4 * g], acc[m][nb][4 * g + 1], acc[m][nb][4 * g + 2],
                          acc[m][nb][4 * g + 3]);
    __syncthreads();
#pragma unroll
    for (int p0 = 0; p0 < 4 * MB; p0 += kCombRows) {
      uint4 o[kCombRows][kMaxTopK], rv[kCombRows];
#pragma unroll
      for (int q = 0; q < kCombRows; ++q) {
        const int rc = min(8 * (p0 + q) + (tid >> 5), nvalid - 1);
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
          // unused ranks (j >= k) repeat the last one's load and are not added
          const int32_t slot = s_slot[rc * k + min(j, k - 1)];
          o[q][j] = *reinterpret_cast<const uint4 *>(a.out + (size_t)slot * a.H + col0);
        }
        rv[q] = a.residual ? *reinterpret_cast<const uint4 *>(
                                 a.residual + (size_t)(row0 + rc) * a.H + col0)
                           : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < kCombRows; ++q) {
        const int r_tile = 8 * (p0 + q) + (tid >> 5);
        if (r_tile >= nvalid) continue;
        const int64_t t = row0 + r_tile;
        const float4 s0 = *reinterpret_cast<const float4 *>(st + r_tile * SP + cc);
        const float4 s1 = *reinterpret_cast<const float4 *>(st + r_tile * SP + cc + 4);
        float v[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
          if (j >= k) break;
          v[0] += f16lo(o[q][j].x); v[1] += f16hi(o[q][j].x); v[2] += f16lo(o[q][j].y);
          v[3] += f16hi(o[q][j].y); v[4] += f16lo(o[q][j].z); v[5] += f16hi(o[q][j].z);
          v[6] += f16lo(o[q][j].w); v[7] += f16hi(o[q][j].w);
        }
        if (a.residual) {
          const uint4 w4 = rv[q];
          v[0] += bf16lo(w4.x); v[1] += bf16hi(w4.x); v[2] += bf16lo(w4.y); v[3] += bf16hi(w4.y);
          v[4] += bf16lo(w4.z); v[5] += bf16hi(w4.z); v[6] += bf16lo(w4.w); v[7] += bf16hi(w4.w);
        }
        *reinterpret_cast<uint4 *>(a.y + (size_t)t * a.H + col0) =
            make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      }
    }
  } else {
    // rows x 256 columns fp16 in slot order: a routed slot pre-weighted by its routing
    // weight, a shared-expert slot (weight 1) as it is; staged through LDS 128 rows at a time.
    // Transposed accumulators (kWT): lane l holds slot row 32m + l%32, and register r the
    // output column 8*(r/4) + 4*(l/32) + r%4 of its 32-column block. Rows are padded by
    // 16 bytes, which spreads the 8-byte writes of 16 rows over all banks.
    constexpr int OP = BNW + 8;
    _Float16 *ot = reinterpret_cast<_Float16 *>(smem);
    float *sw = reinterpret_cast<float *>(smem + (kPreSw ? kSwOff : BM * OP * 2));
    static_assert(BM * OP * 2 + kMaxMB * 32 * 4 <= kSwOff, "epilogue staging");
    // the routed weights are in LDS already (kPreSw); the shared expert's rows have weight 1
    if (!kPreSw || e == a.E)
      if (tid < 32 * MB) sw[tid] = tid < nvalid ? (e < a.E ? a.slot_w[slot0 + tid] : 1.0f) : 0.f;
#pragma unroll
    for (int m0 = 0; m0 < MB; m0 += 4) {
      // sw is written; the previous round's rows have left
      if (!kPreSw || e == a.E || m0 > 0) __syncthreads();
#pragma unroll
      for (int m = m0; m < (MB < m0 + 4 ? MB : m0 + 4); ++m) {
        const int row = 32 * m + col;
        const float wv = sw[row];
        _Float16 *orow = ot + (row - 32 * m0) * OP + 64 * wave + rq4;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<uint2 *>(orow + 32 * nb + 8 * g) =
                make_uint2(mul_pack_f16x2(wv, acc[m][nb][4 * g], acc[m][nb][4 * g + 1]),
                           mul_pack_f16x2(wv, acc[m][nb][4 * g + 2], acc[m][nb][4 * g + 3]));
      }
      __syncthreads();
      const int r1 = min(nvalid, 32 * (m0 + 4));
      for (int rr = 32 * m0 + (tid >> 5); rr < r1; rr += 8)
        *reinterpret_cast<uint4 *>(a.out + (size_t)(slot0 + rr) * a.H + n_tile * BNW +
                                   8 * (tid & 31)) =
            *reinterpret_cast<const uint4 *>(ot + (rr - 32 * m0) * OP + 8 * (tid & 31));
    }
  }
  if (tk && tid == 0) *reinterpret_cast<int32_t *>(smem + kTicketOff) = tn;
}

// N tile n_tile of entry m_tile of the tile map
template <bool kGateUp, bool kX>
MOE_DEV bool grouped_item(const GroupedArgs &a, uint8_t *smem, int m_tile, int n_tile, int wave,
                          int32_t *tk = nullptr) {
  const int2 tile = a.tiles[m_tile];
  const int tx = __builtin_amdgcn_readfirstlane(tile.x), row0 = __builtin_amdgcn_readfirstlane(tile.y);
  const int e = tx & 0xFFFF, nvalid = tx >> 16;
  // the shared expert's down projection runs in its own launch with the combine fused
  if (!kGateUp && a.fused_combine && e == a.E) return false;
  // load-adaptive height: only the 32-row blocks that hold rows (all four when fixed)
  switch (a.fixed_mb ? 4 : (nvalid + 31) >> 5) {
    case 1: grouped_tile<kGateUp, 1, kX>(a, smem, e, row0, nvalid, n_tile, wave, tk); break;
    case 2: grouped_tile<kGateUp, 2, kX>(a, smem, e, row0, nvalid, n_tile, wave, tk); break;
    case 3: grouped_tile<kGateUp, 3, kX>(a, smem, e, row0, nvalid, n_tile, wave, tk); break;
    case 4: grouped_tile<kGateUp, 4, kX>(a, smem, e, row0, nvalid, n_tile, wave, tk); break;
    default: grouped_tile<kGateUp, 5, kX>(a, smem, e, row0, nvalid, n_tile, wave, tk); break;
  }
  return true;
}

template <bool kGateUp, bool kX>
MOE_DEV void grouped_body(const GroupedArgs &a, uint8_t *smem) {
  // XCD-aware tile order: workgroup ids are dealt round-robin over the 8 XCDs; this map
  // gives each XCD all N tiles of one M tile back to back, so the activation rows of a
  // tile are fetched into that XCD's L2 once.
  const int nN = kGateUp ? a.I / (BNW / 2) : a.H / BNW;
  const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
  const int n_tile = j % nN, m_tile = (j / nN) * 8 + xcd;
  if (m_tile >= *a.n_tiles) return;
  grouped_item<kGateUp, kX>(a, smem, m_tile, n_tile,
                            __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6));
}

template <bool kGateUp>
__global__ __launch_bounds__(256, 2) void k_grouped(GroupedArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  grouped_body<kGateUp, false>(a, smem);
}

// Down projection of the shared expert with the weighted combine in its epilogue: token tiles
// of 64 rows (the shared expert's slots kT + t), every N tile of 256 output columns. XCD-aware
// order as in grouped_body. Runs after the routed down projection (stream order).
__global__ __launch_bounds__(256, 2) void k_shared_down_combine(GroupedArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  const int nN = a.H / BNW;
  const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
  const int n_tile = j % nN, m_tile = (j / nN) * 8 + xcd;
  const int row0 = 64 * m_tile;
  if (row0 >= a.T) return;
  const int nvalid = min(64, (int)(a.T - row0));
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (nvalid > 32)
    grouped_tile<false, 2, false, true>(a, smem, a.E, row0, nvalid, n_tile, wave);
  else
    grouped_tile<false, 1, false, true>(a, smem, a.E, row0, nvalid, n_tile, wave);
}

// gate/up and down of every tile in one persistent launch. The down GEMM of a tile needs all
// of its rows' h, so as two launches the down work waits for the whole gate/up grid, and the
// gate/up grid's last, partly filled round of workgroups leaves CUs idle. Here the tiles are
// dealt to one queue per XCD in runs of kRun consecutive tiles of the map (run j to queue
// j mod Q, Q queues), so that the tiles of an expert with several tiles mostly share one L2
// for its weights; a queue holds first every gate/up item (tile, N tile), then every down
// item. A workgroup
// serves its own XCD's queue first (q is read from the XCC_ID register), so a tile's x rows,
// weights and h mostly stay in one L2; once that queue is empty it serves the next queues in
// turn, because equal shares of work do not finish together on every XCD. A workgroup takes
// the next item of a queue with an atomic ticket, so only running workgroups hold work. A
// gate/up item writes its h rows through to memory, waits until the stores are acknowledged
// and then counts itself done on the tile; a down item first waits for its tile's count to
// reach the gate/up N tiles. Tickets and counts are system-scope atomics and loads, performed
// in memory, so workgroups on any XCD see the same values; a down item's h loads go through
// its own L2 and L1, which hold no copy of those rows: nothing in the launch reads them
// before they are complete, and the caches hold nothing older from before the launch.
// Deadlock-free: gate/up items wait for nothing, and a down item waits only for gate/up items
// of its queue with earlier tickets, all taken by running workgroups. The waits are bounded
// anyway (kSpinTicks of the 100 MHz clock, then the flag at kSyncErr is raised and the item
// computed as it stands).
constexpr uint64_t kSpinTicks = 50000000ull;  // 0.5 s
constexpr int kRun = 4;  // consecutive tiles of the map dealt to one queue

__global__ __launch_bounds__(256, 2) void k_grouped_fused(GroupedArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const bool lead = threadIdx.x == 0;
  const int nq = a.n_queues;
  const int nt = *a.n_tiles;
  const int nNg = a.I / (BNW / 2), nNd = a.H / BNW;
  int32_t *s_t = reinterpret_cast<int32_t *>(smem + kTicketOff);  // the next ticket
  // the queue served now (this XCD's first), and the queues not yet found empty
  int cq = (int)(__builtin_amdgcn_s_getreg(20 | (31 << 11)) & (uint32_t)(nq - 1)), left = nq;
  if (lead)
    *s_t = __hip_atomic_fetch_add(a.sync + kSyncQStride * cq, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_SYSTEM);
  __syncthreads();
  int t = __builtin_amdgcn_readfirstlane(*s_t);  // uniform: addresses stay scalar
  __syncthreads();
  while (true) {
    // tiles of queue cq: runs of kRun consecutive tiles of the map, run j to queue j % nq
    const int per_round = nq * kRun, rounds = nt / per_round;
    const int ntq = rounds * kRun + min(kRun, max(0, nt - rounds * per_round - cq * kRun));
    const int n_gu = ntq * nNg, n_all = n_gu + ntq * nNd;
    if (t >= n_all) {
      // queue cq is empty: the next one
      if (--left == 0) break;
      cq = (cq + 1) & (nq - 1);
      if (lead)
        *s_t = __hip_atomic_fetch_add(a.sync + kSyncQStride * cq, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
      __syncthreads();
      t = __builtin_amdgcn_readfirstlane(*s_t);
      __syncthreads();
      continue;
    }
    // The arguments are read through an opaque copy of the kernel-argument pointer, so that
    // the compiler loads them per item (scalar loads) instead of holding every field and
    // what it derives from them in SGPRs across the loop.
    typedef const GroupedArgs __attribute__((address_space(4))) KArgs;
    KArgs *ap = (KArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    const GroupedArgs &ai = *(const GroupedArgs *)ap;
    int32_t *tk = ai.sync + kSyncQStride * cq;
    bool ran;
    if (t < n_gu) {
      const int i = t / nNg, m = (i / kRun) * (nq * kRun) + cq * kRun + i % kRun;
      ran = grouped_item<true, false>(ai, smem, m, t - i * nNg, wave, tk);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's h stores are in memory
      __syncthreads();
      if (lead)
        __hip_atomic_fetch_add(ai.sync + kSyncDone + m, 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
    } else {
      const int u = t - n_gu, i = u / nNd, m = (i / kRun) * (nq * kRun) + cq * kRun + i % kRun;
      if (lead) {
        int32_t *done = ai.sync + kSyncDone + m, *err = ai.sync + kSyncErr;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) < nNg) {
          if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)) break;
          if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
            __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      __syncthreads();
      ran = grouped_item<false, false>(ai, smem, m, u - i * nNd, wave, tk);
    }
    // a skipped item (the shared expert's down tiles, whose launch is the fused combine)
    // took no ticket
    if (!ran && lead)
      *s_t = __hip_atomic_fetch_add(tk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __syncthreads();  // the next ticket is in LDS
    t = __builtin_amdgcn_readfirstlane(*s_t);
    __syncthreads();  // every wave has read it before it is replaced
  }
}

template <bool kGateUp>
__global__ __launch_bounds__(256, 1) void k_grouped_x(GroupedArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kXSmemBytes];
  grouped_body<kGateUp, true>(a, smem);
}

// ---- separate dequantisation pass (ablation) -------------------------------------------
// One workgroup per (64-row block, K step) of one expert: thread (kk, l) expands the code
// word of substep kk of lane l for both column blocks with the same packed dequantisation
// the GEMM runs in registers, so the expanded operands are bit-identical to the fused ones.
// Experts that received no rows are skipped (the shared expert always has T rows).
template <bool kGateUp>
__global__ __launch_bounds__(256) void k_expand(GroupedArgs a) {
  const int e = blockIdx.y;
  if (e < a.E && a.offsets[e + 1] == a.offsets[e]) return;
  const int K = kGateUp ? a.H : a.I;
  const int nb = kGateUp ? 2 * a.I / 64 : a.H / 64;
  const int ns = K / BK, ns4 = (ns + 3) / 4;
  const int blk = blockIdx.x / ns, st = blockIdx.x % ns;
  const int kk = threadIdx.x >> 6, lane = threadIdx.x & 63, bn = lane & 31, bh = lane >> 5;
  const uint8_t *tq = (kGateUp ? a.wt.w13_t : a.wt.w2_t) +
                      (((size_t)e * nb + blk) * ns + st) * 2048 + 32 * bn + 16 * bh + 4 * kk;
  const uint16_t *tsb = (kGateUp ? a.wt.w13_tsb : a.wt.w2_tsb) +
                        (((size_t)e * nb + blk) * ns4 + st / 4) * 512 + 8 * bn + 2 * (st & 3);
  uint16_t *dst = const_cast<uint16_t *>(kGateUp ? a.w13_x : a.w2_x) +
                  (((size_t)e * nb + blk) * ns + st) * 4096 + kk * 512 + 8 * lane;
  const f16x2_t q16 = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(tq + c * 1024);
    const f16x2_t sc = f16_pair_from_bf16(tsb[256 * c]), bi = f16_pair_from_bf16(tsb[256 * c + 1]);
    *reinterpret_cast<uint4 *>(dst + c * 2048) = dequant8_pk_q(w, sc, sc * q16, bi);
  }
}

size_t expanded_bytes(int n_mat, int rows, int K) { return (size_t)n_mat * rows * K * 2; }

hipError_t launch_expand(const GroupedArgs &a, hipStream_t s) {
  const unsigned ne = (unsigned)(a.E + (a.S ? 1 : 0));
  MOE_LAUNCH("k_expand_gateup", (k_expand<true>), dim3((2 * a.I / 64) * (a.H / BK), ne),
             dim3(256), 0, s, a);
  MOE_LAUNCH("k_expand_down", (k_expand<false>), dim3((a.H / 64) * (a.I / BK), ne), dim3(256),
             0, s, a);
  return hipSuccess;
}

static unsigned grouped_grid(int max_tiles, int nN) {
  const int mt_pad = (max_tiles + 7) / 8 * 8;
  return (unsigned)(mt_pad * nN);
}

hipError_t launch_grouped_gateup(const GroupedArgs &a, hipStream_t s) {
  const dim3 g(grouped_grid(a.max_tiles, a.I / (BNW / 2)));
  if (a.w13_x)
    MOE_LAUNCH("k_grouped_gateup_x", (k_grouped_x<true>), g, dim3(256), 0, s, a);
  else
    MOE_LAUNCH("k_grouped_gateup", (k_grouped<true>), g, dim3(256), 0, s, a);
  return hipSuccess;
}

hipError_t launch_shared_down_combine(const GroupedArgs &a, hipStream_t s) {
  const int mt = (int)((a.T + 63) / 64);
  const dim3 g((unsigned)((mt + 7) / 8 * 8 * (a.H / BNW)));
  MOE_LAUNCH("k_shared_down_combine", k_shared_down_combine, g, dim3(256), 0, s, a);
  return hipSuccess;
}

hipError_t launch_grouped_fused(const GroupedArgs &a, hipStream_t s) {
  if (!a.sync || a.n_queues < 1 || a.n_queues > kMaxQueues || (a.n_queues & (a.n_queues - 1)))
    return hipErrorInvalidValue;
  // two resident workgroups per CU, 32 CUs per XCD
  MOE_LAUNCH("k_grouped_fused", k_grouped_fused, dim3((unsigned)(64 * a.n_queues)), dim3(256),
             0, s, a);
  return hipSuccess;
}

hipError_t launch_grouped_down(const GroupedArgs &a, hipStream_t s) {
  const dim3 g(grouped_grid(a.max_tiles, a.H / BNW));
  if (a.w2_x)
    MOE_LAUNCH("k_grouped_down_x", (k_grouped_x<false>), g, dim3(256), 0, s, a);
  else
    MOE_LAUNCH("k_grouped_down", (k_grouped<false>), g, dim3(256), 0, s, a);
  return hipSuccess;
}

}  // namespace moe
