// kernels.h -- internal launch interface between the host library and the kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Kernel timing hook (host side, implemented in moe_api.hip). When profiling is on it
// hands out a start/stop event pair bound to the next dispatch (hipExtLaunchKernel
// timestamps the kernel itself, not the queue around it); otherwise it returns false.
bool prof_events(const char *name, hipEvent_t *start, hipEvent_t *stop);

#define MOE_LAUNCH(name, kern, grid, block, shm, stream, ...)                               \
  do {                                                                                      \
    hipEvent_t moe_ev_a_ = nullptr, moe_ev_b_ = nullptr;                                    \
    if (::moe::prof_events(name, &moe_ev_a_, &moe_ev_b_))                                   \
      hipExtLaunchKernelGGL(kern, grid, block, shm, stream, moe_ev_a_, moe_ev_b_, 0,         \
                            __VA_ARGS__);                                                   \
    else                                                                                    \
      hipLaunchKernelGGL(kern, grid, block, shm, stream, __VA_ARGS__);                      \
    const hipError_t moe_err_ = hipGetLastError();                                          \
    if (moe_err_ != hipSuccess) return moe_err_;                                            \
  } while (0)

// Routing blocks per chunk of the two-level count scan, and the call size (in routing blocks)
// above which it is used: the grouping kernel's reads then grow with T instead of T^2, at the
// price of one more launch (k_chunk_sum).
constexpr int kChunkBlocks = 64;
constexpr int kChunkFromBlocks = 4 * kChunkBlocks;
struct RouteArgs {
  bool bf16;
  const void *x;
  const float *router_w, *router_b;
  int64_t T;
  int H, E, k, S;
  int I = 0;              // expert intermediate size (sizes the tile-height choice)
  float *logits;          // fp32 path: [T, E]; bf16 path: kRouterParts partial sums [4][T, E]
  uint16_t *router_planes;  // fp16 split of the router weights in B-fragment order (bf16 path)
  bool planes_ready;        // router_planes already hold the split (packed layer)
  int32_t *ids;           // [T, k]
  float *w;               // [T, k]
  int32_t *blk;           // [NB, E] per-block counts, then per-block bases
  int32_t *chunk = nullptr;  // [ceil(NB / kChunkBlocks), E] per-chunk counts; set (by the
                             // host) only when NB > kChunkFromBlocks
  int32_t *offsets;       // [E + 2]
  int32_t *counts_user;   // [E] or null
  int32_t *offsets_user;  // [E + 1] or null
  int32_t *sorted_tok;    // [k T]
  int32_t *slot_of;       // [T, k]
  float *slot_w;          // [k T] routing weight of each slot (prefill only)
  uint16_t *x16;          // [T, H] fp16 copy of x for the MFMA path (or null)
  int2 *tiles;            // [max tiles]: (group, first row)
  int32_t *n_tiles;       // [1]
  int tile_shift = 0;     // grouped-GEMM tile height: 0 = chosen from the load on the GPU,
                          // else fixed at 2^tile_shift rows (5..7)
  int32_t *sync = nullptr;  // [n_sync] work-queue words of k_grouped_fused, zeroed by k_group
  int n_sync = 0;
};

// Router, top-k and per-block histogram (launch_route_topk), then one kernel that forms the
// group offsets and tile map and scatters the assignments (k_group).
hipError_t launch_route_prefill(const RouteArgs &a, hipStream_t s);
hipError_t launch_route_topk(const RouteArgs &a, hipStream_t s);
// The scatter alone, from offsets, per-block bases and tile map already in memory (the
// host-routing ablation uploads them).
hipError_t launch_route_scatter(const RouteArgs &a, hipStream_t s);

struct ExpertWeights {
  const uint8_t *w13_q, *w2_q;     // int4 codes, interchange layout
  const uint16_t *w13_s, *w13_b;   // bf16 scale / bias
  const uint16_t *w2_s, *w2_b;
  const uint8_t *w13_t, *w2_t;     // int4 codes, tiled layout (moe_pack_weights)
  const uint16_t *w13_tsb, *w2_tsb;  // tiled {scale, bias} pairs
  const float *w13_f, *w2_f;       // fp32 weights (MOE_W_F32)
};

// Repack of one stacked int4 matrix (n_mat experts of rows x K) into the tiled layout.
struct PackArgs {
  const uint8_t *q;
  const uint16_t *sc, *bi;
  int rows, K, n_mat, inter;
  bool gate_up;
  uint8_t *t;
  uint16_t *tsb;
};
size_t tiled_code_bytes(int n_mat, int rows, int K);
size_t tiled_sb_bytes(int n_mat, int rows, int K);
hipError_t launch_pack(const PackArgs &a, hipStream_t s);
// The router's two fp16 planes in B-fragment order (see k_router_split); bytes for E experts.
constexpr int kRouterParts = 4;  // partial logit arrays of the bf16 router (quarters of H)
size_t router_frag_bytes(int E, int H);
hipError_t launch_router_split(const float *W, int E, int H, uint16_t *planes, hipStream_t s);

// Grouped int4 GEMMs of the prefill path (fp16 operands, fp32 accumulation).
struct GroupedArgs {
  const uint16_t *x16;        // [T, H] fp16
  const int32_t *sorted_tok;  // [k T]
  const float *slot_w;        // [k T]
  const int32_t *offsets;     // [E + 2]
  const int2 *tiles;          // (group | rows << 16, first row) per tile
  const int32_t *n_tiles;
  int max_tiles;
  int64_t T;
  int H, I, E, k;
  ExpertWeights wt;
  uint16_t *h16;   // [(k+S) T, I] fp16, slot order
  uint16_t *out;   // [k T, H] fp16, slot order: routed slots already scaled by the
                   // routing weight
  // Weighted combine fused into the shared expert's down projection (S == 1): the routed
  // down launch skips the shared expert's tiles and launch_shared_down_combine writes y.
  int fused_combine = 0;
  const int32_t *slot_of = nullptr;   // [T, k]
  const uint16_t *residual = nullptr; // [T, H] bf16 or null
  uint16_t *y = nullptr;              // [T, H] bf16
  // Ablation switches (moe_prefill_ablation); the product path leaves them unset.
  int fixed_mb = 0;        // every tile multiplies all four 32-row blocks
  int S = 0;               // shared experts (launch_expand only)
  // fp16 weights expanded by launch_expand (tiled order, see expanded_bytes); when set, the
  // GEMMs read them instead of the int4 codes
  const uint16_t *w13_x = nullptr, *w2_x = nullptr;
  // Work queues of the fused gate/up + down launch (launch_grouped_fused): sync_words words,
  // zero at launch; n_queues = the device's XCDs (a power of two, at most kMaxQueues).
  int32_t *sync = nullptr;
  int n_queues = 0;
};
// Work-queue words of k_grouped_fused: queue q's ticket at kSyncQStride * q (one 256-byte
// line each), the give-up flag of the bounded waits at kSyncErr, then one completion counter
// per tile of the tile map.
constexpr int kMaxQueues = 8, kSyncQStride = 64, kSyncErr = kMaxQueues * kSyncQStride;
constexpr int kSyncDone = kSyncErr + 64;
inline size_t sync_words(int max_tiles) { return (size_t)kSyncDone + (size_t)max_tiles; }
hipError_t launch_grouped_gateup(const GroupedArgs &a, hipStream_t s);
hipError_t launch_grouped_down(const GroupedArgs &a, hipStream_t s);
// gate/up and down in one persistent launch (a.sync set): one queue of tiles per XCD (runs of
// consecutive tiles), all gate/up work first, a down tile starting once its rows' h is
// complete; workgroups serve their own XCD's queue, then the others.
hipError_t launch_grouped_fused(const GroupedArgs &a, hipStream_t s);
hipError_t launch_shared_down_combine(const GroupedArgs &a, hipStream_t s);
// Separate dequantisation pass: every expert that received rows (and the shared expert)
// expanded to fp16, [E+S][R/64][K/64][2 column blocks][4 substeps][64 lanes][8], the B
// operand registers of the grouped GEMM in the order it reads them.
size_t expanded_bytes(int n_mat, int rows, int K);
hipError_t launch_expand(const GroupedArgs &a, hipStream_t s);

// Weighted combine of the slot-ordered expert outputs back to token order.
// (layers without a shared expert)
struct CombineArgs {
  const uint16_t *out;       // [k T, H] fp16: weighted routed outputs in slot order
  const int32_t *slot_of;    // [T, k]
  const uint16_t *residual;  // [T, H] or null
  uint16_t *y;               // [T, H]
  int64_t T;
  int H, k;
};
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);

// Per-token GEMV path (batch-1 decode; also the fp32-weight layers).
struct TokenArgs {
  bool bf16;                 // activation dtype (int4 weights imply bf16)
  bool int4;
  const void *x;             // [T, H]
  const int32_t *ids;        // [T, k]
  const float *w;            // [T, k]
  const void *residual;      // [T, H] or null
  void *y;                   // [T, H]
  float *h;                  // [T, k+S, I] fp32
  int64_t T;
  int H, I, E, k, S;
  ExpertWeights wt;
};
hipError_t launch_token_experts(const TokenArgs &a, hipStream_t s);

// Batch-1 layer in three kernels (hidden 2048, intermediate 512, int4); the same kernels'
// small-T variant takes T <= kSmallT tokens.
constexpr int kSmallT = 8;
struct DecodeArgs {
  const uint16_t *x;          // [H] bf16
  const float *router_w, *router_b;
  ExpertWeights wt;
  const uint16_t *residual;   // [H] or null
  uint16_t *y;                // [H]
  float *z;                   // [E] logits
  float *h;                   // [k+S, I] fp32
  int32_t *sel_ids;           // [k] selected experts, rank order (largest logit first);
                              // small-T: [T, k] in ascending id order
  float *sel_z;               // [k] their logits; small-T: [T, k] their routing weights
  int T;                      // tokens (small-T path; 1 for decode): x [T,H], z [T,E],
                              // h [T,k+S,I], y and residual [T,H]
  int sel_is_w;               // sel_z holds routing weights, not logits
  int H, I, E, k, S;
  // when set, the layer reads RMSNorm(x) (unit gain, fp64, rounded once to bf16) instead of
  // x: k_dec_a forms it and stores it in xn [H] for k_dec_b; the residual is still the
  // caller's (un-normalised) pointer
  int norm;
  float eps;
  uint16_t *xn;
};
bool decode_gemv_supported(int H, int I, int E, int k, int S, bool int4);
hipError_t launch_decode_gemv(const DecodeArgs &a, hipStream_t s);
hipError_t launch_small_t(const DecodeArgs &a, hipStream_t s);

// Measurement aids: the decode kernels' weight loads without their arithmetic (part 0:
// router, 1: gate/up, 2: down; experts from a.sel_ids), and a dense MFMA loop of
// kMfmaCeilingWG workgroups x 4 waves x iters x 8 v_mfma_f32_32x32x16_f16.
hipError_t launch_read_ceiling(const DecodeArgs &a, int part, uint32_t *sink, hipStream_t s);
constexpr int kMfmaCeilingWG = 512;
hipError_t launch_mfma_ceiling(int iters, int low_entropy, uint32_t *sink, hipStream_t s);

hipError_t launch_rmsnorm(const void *h, int64_t T, int H, float eps, bool bf16, void *out,
                          hipStream_t s);

// Decode attention of one token over a grouped-query KV cache (bf16, head dimension 256).
constexpr int kAttnMaxSlots = 512;  // workgroups the cache blocks are spread over, at most
struct AttnArgs {
  const uint16_t *q;          // [n_q, 256] bf16
  const uint16_t *k, *v;      // head g's row t at g * head_stride + t * 256 (bf16)
  int64_t head_stride;        // elements
  int64_t ctx;                // cached positions (>= 1)
  int64_t tps;                // positions per block (multiple of 32)
  int n_split;                // blocks
  int n_q, G;                 // query heads, query heads per KV head
  float scale_log2;           // score scale times log2(e)
  float *part_acc;            // [n_split, n_q, 256] unnormalised block sums
  float *part_m, *part_l;     // [n_split, n_q] block maxima (exp2 domain) and sums
  uint16_t *out;              // [n_q, 256] bf16
};
bool attn_supported(int n_q, int n_kv, int D);
void attn_plan(int64_t ctx, int n_groups, int *n_split, int64_t *tps);
// heads_per_group: G (query heads of a KV head share a workgroup) or 1 (one per head)
hipError_t launch_attn_decode(const AttnArgs &a, int heads_per_group, hipStream_t s);

// Gated DeltaNet recurrence over T tokens (d_k = d_v = 128), state fp32 in and out.
struct GdnArgs {
  const uint16_t *q, *k;        // [T, n_k, 128] bf16
  const uint16_t *v;            // [T, n_v, 128] bf16
  const float *alpha, *beta;    // [T, n_v]
  int64_t T;                    // >= 1
  int n_k, n_v;
  float *state;                 // [n_v, 128, 128]: S_0 in, S_T out
  uint16_t *out;                // [T, n_v, 128] bf16
  float *ws = nullptr;          // chunked form: per (value head, chunk) factors and tables
  int nch = 0;                  // chunks of 32 tokens
};
bool gdn_supported(int n_k, int n_v, int d_k, int d_v);
hipError_t launch_gdn_scan(const GdnArgs &a, hipStream_t s);
size_t gdn_chunk_ws_bytes(int64_t T, int n_v);
hipError_t launch_gdn_chunked(const GdnArgs &a, hipStream_t s);

}  // namespace moe
