// pack.hip -- one-time repack of int4 expert weights into the tiled layout of the
// grouped GEMMs.
//
// "Optimizing On-Device Inference for Apple Silicon", section "Dequantize weights during
// matrix multiplication": the weights stay 4-bit with one bf16 scale and bias per 64
// weights; only their order in memory changes, so that every load a GEMM wave issues
// for a K step is one contiguous 1 KB block (32 rows x 32 code bytes) instead of 32
// rows spread over the row-major array, and the scales and biases of four steps arrive
// as one 1 KB block (64 rows x 4 groups x {scale, bias}).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// Source row of row r (0..63) of tiled block j. The gate/up matrix pairs gate row 32j + r
// with up row I + 32j + r in one block, so one GEMM wave's two B operands share a block.
MOE_DEV int tiled_src_row(bool gate_up, int inter, int j, int r) {
  if (gate_up) return r < 32 ? 32 * j + r : inter + 32 * j + (r - 32);
  return 64 * j + r;
}

// One thread per 16 output bytes: (expert e, block j, step s, row r, half h).
__global__ __launch_bounds__(256) void k_pack_codes(const uint8_t *__restrict__ q, int rows,
                                                    int K, int n_mat, bool gate_up, int inter,
                                                    uint8_t *__restrict__ t) {
  const int nb = rows / 64, ns = K / 64;
  const size_t total = (size_t)n_mat * nb * ns * 128;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int h = (int)(i & 1), r = (int)((i >> 1) & 63);
    size_t rest = i >> 7;
    const int s = (int)(rest % ns);
    rest /= ns;
    const int j = (int)(rest % nb);
    const size_t e = rest / nb;
    const size_t row = e * rows + tiled_src_row(gate_up, inter, j, r);
    const uint4 v = *reinterpret_cast<const uint4 *>(q + row * (K / 2) + 32 * s + 16 * h);
    *reinterpret_cast<uint4 *>(t + 16 * i) = v;
  }
}

// One thread per (expert e, block j, 4-group step s4, row r): 4 x {scale, bias}.
__global__ __launch_bounds__(256) void k_pack_scales(const uint16_t *__restrict__ sc,
                                                     const uint16_t *__restrict__ bi,
                                                     int rows, int K, int n_mat, bool gate_up,
                                                     int inter, uint16_t *__restrict__ tsb) {
  const int nb = rows / 64, ng = K / 64, ns4 = (ng + 3) / 4;
  const size_t total = (size_t)n_mat * nb * ns4 * 64;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(i & 63);
    size_t rest = i >> 6;
    const int s4 = (int)(rest % ns4);
    rest /= ns4;
    const int j = (int)(rest % nb);
    const size_t e = rest / nb;
    const size_t row = e * rows + tiled_src_row(gate_up, inter, j, r);
    uint16_t out[8];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * s4 + gi;
      out[2 * gi] = g < ng ? sc[row * ng + g] : 0;
      out[2 * gi + 1] = g < ng ? bi[row * ng + g] : 0;
    }
    uint4 v;
    v.x = out[0] | ((uint32_t)out[1] << 16);
    v.y = out[2] | ((uint32_t)out[3] << 16);
    v.z = out[4] | ((uint32_t)out[5] << 16);
    v.w = out[6] | ((uint32_t)out[7] << 16);
    *reinterpret_cast<uint4 *>(tsb + 8 * i) = v;
  }
}

}  // namespace

size_t tiled_code_bytes(int n_mat, int rows, int K) { return (size_t)n_mat * rows * (K / 2); }

size_t tiled_sb_bytes(int n_mat, int rows, int K) {
  return (size_t)n_mat * (rows / 64) * ((K / 64 + 3) / 4) * 64 * 16;
}

hipError_t launch_pack(const PackArgs &a, hipStream_t s) {
  const unsigned grid = 2048;
  MOE_LAUNCH("k_pack_codes", k_pack_codes, dim3(grid), dim3(256), 0, s, a.q, a.rows, a.K,
             a.n_mat, a.gate_up, a.inter, a.t);
  MOE_LAUNCH("k_pack_scales", k_pack_scales, dim3(grid), dim3(256), 0, s, a.sc, a.bi, a.rows,
             a.K, a.n_mat, a.gate_up, a.inter, a.tsb);
  return hipSuccess;
}

}  // namespace moe
