/* moe.h -- C ABI of the routed-expert MoE layer for MI355X (gfx950).
 *
 * The layer: a router scores E experts per token, the k best are kept with softmax
 * weights renormalised over the selection, one shared expert is added for every
 * token, and every expert is a SwiGLU MLP whose weights stay int4 (groups of 64, one
 * bf16 scale and one bf16 bias per group) until they are dequantised on chip
 * ("Optimizing On-Device Inference for Apple Silicon", sections "Qwen creates three
 * distinct workload shapes" and "Dequantize weights during matrix multiplication").
 *
 * Conventions for every call below:
 *   - Pointers named x, y, residual, router_*, w*_*, ws and the moe_route_out fields
 *     are DEVICE pointers; moe_layer / moe_route_out structs and `bytes` are HOST.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls
 *     only enqueue work on it: they never synchronise the host and never copy device
 *     memory to the host, so a whole layer can be captured into a HIP graph (the one
 *     exception is the host-routing ablation, which exists to measure exactly that).
 *   - The caller owns all memory (inputs, outputs, weights, workspace). The library
 *     never allocates or frees device memory.
 *   - Errors are detected on the host before anything is enqueued (except MOE_E_HIP,
 *     a launch failure). A failing call returns a negative moe_status, enqueues
 *     nothing (or nothing further) and sets a thread-local message readable with
 *     moe_last_error(). Nothing throws across the ABI.
 *   - Calls that share one workspace must not overlap in time (same stream is fine).
 */
#ifndef ROUTED_EXPERT_MOE_H
#define ROUTED_EXPERT_MOE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

typedef enum {
  MOE_OK = 0,
  MOE_E_INVALID = -1,      /* null pointer, bad size, inconsistent descriptor */
  MOE_E_UNSUPPORTED = -2,  /* valid but outside what the kernels implement */
  MOE_E_WORKSPACE = -3,    /* workspace smaller than moe_workspace_bytes() */
  MOE_E_HIP = -4           /* a HIP call or kernel launch failed (no device, ...) */
} moe_status;

typedef enum { MOE_W_F32 = 0, MOE_W_INT4_G64 = 1 } moe_w_format;
typedef enum { MOE_ACT_F32 = 0, MOE_ACT_BF16 = 1 } moe_act_dtype;

/* One layer. Experts 0..E-1 are routed; with n_shared == 1 the shared expert is
 * stacked after them as expert index E.
 *   router_w  float [E, H] row-major;  router_b  float [E] or NULL (added to logits)
 *   MOE_W_INT4_G64 (requires act_dtype == MOE_ACT_BF16), interchange layout:
 *     w13_q uint8 [E+S, 2I, H/2]: row r holds the gate projection for r < I and the up
 *           projection for r >= I; byte j of a row holds element 2j in its low nibble
 *           and element 2j+1 in its high nibble (unsigned codes 0..15)
 *     w13_s, w13_b  bf16 bit patterns [E+S, 2I, H/64]: scale and bias of each group of
 *           64 consecutive elements of a row; weight = scale * code + bias
 *     w2_q uint8 [E+S, H, I/2], w2_s / w2_b bf16 [E+S, H, I/64]: output projection
 *     w13_t, w13_tsb, w2_t, w2_tsb: the same weights in the tiled layout written by
 *           moe_pack_weights (NULL until packed); moe_prefill needs them
 *   MOE_W_F32 (requires act_dtype == MOE_ACT_F32):
 *     w13_q float [E+S, 2I, H], w2_q float [E+S, H, I]; the other weight pointers unused
 * Supported: 1 <= k <= 8, k <= E <= 256, S in {0,1}; H % 64 == 0, I % 64 == 0,
 * and for int4 additionally H % 256 == 0 and I % 128 == 0. Pointers to codes, tiled
 * arrays, fp32 weights, activations and the workspace must be 16-byte aligned; int4
 * scale and bias pointers 4-byte aligned. Int4 weights are rebuilt in fp16 on the GPU
 * (prefill path): scales, biases, weights, x and h must stay below 65504 in magnitude
 * (results are unspecified otherwise). A weight is rebuilt as the fp16 rounding of the exact
 * scale * code + bias when its group's scale is 0 or |scale| >= 2^-13 and its bias is 0 or
 * |bias| >= 2^-14; in a group outside that range the rebuilt weight carries an extra
 * absolute error of at most 2^-17 (fp16 subnormals). The decode kernels use the scales and
 * biases in fp32 and have no such range. */
typedef struct {
  int32_t abi_version;  /* must be MOE_ABI_VERSION */
  int32_t hidden, inter, n_experts, top_k, n_shared;
  int32_t w_format, act_dtype;
  const float *router_w;
  const float *router_b;
  const void *w13_q, *w13_s, *w13_b;
  const void *w2_q, *w2_s, *w2_b;
  const void *w13_t, *w13_tsb, *w2_t, *w2_tsb;
  /* router_w split into two fp16 planes, hi = fp16(w) and lo = fp16((w - hi) * 2048), so
   * w = hi + lo / 2048 to about 22 bits (router weights must be below 65504 in magnitude),
   * stored in the matrix-core operand order the prefill router loads directly:
   *   fp16 [E_pad / 32][H / 16][2 planes][64 lanes][8]  (E_pad = E rounded up to 128)
   * where lane l of (column block c, step s) holds expert 32c + l % 32 at positions
   * 16s + 8 (l / 32) .. +7 of the row (zero past E). Written by moe_pack_weights, or NULL:
   * then the prefill router splits router_w into the workspace on every call. */
  const void *router_planes;
} moe_layer;

/* Routing results, all caller-owned device buffers of int32 / float:
 *   topk_ids  [T, k]  selected expert ids of each token in ascending id order
 *   topk_w    [T, k]  matching weights (softmax of the selected logits, sum 1)
 *   counts    [E]     assignments per routed expert
 *   offsets   [E+1]   exclusive prefix sum of counts; offsets[E] = k*T
 *   sorted_tok[k*T]   token of each slot; slots of expert e are
 *                     offsets[e] .. offsets[e+1]-1, tokens ascending within an expert
 *   slot_of   [T, k]  slot of assignment (t, j), i.e. sorted_tok[slot_of[t,j]] == t */
typedef struct {
  int32_t *topk_ids;
  float *topk_w;
  int32_t *counts;
  int32_t *offsets;
  int32_t *sorted_tok;
  int32_t *slot_of;
} moe_route_out;

/* ABI version compiled into the library. */
int32_t moe_abi_version(void);

/* Message of the last failing call on this thread ("" if none). Host string owned by
 * the library, valid until the next call on this thread. */
const char *moe_last_error(void);

/* Workspace size in bytes for calls with up to max_tokens tokens (host out param).
 * No call needs the workspace to hold any particular contents on entry. */
moe_status moe_workspace_bytes(const moe_layer *layer, int64_t max_tokens, size_t *bytes);

/* Bytes of device memory moe_pack_weights needs for an int4 layer (host out param). */
moe_status moe_pack_bytes(const moe_layer *layer, size_t *bytes);

/* One-time repack of an int4 layer's expert weights into the tiled layout read by the
 * grouped GEMMs of moe_prefill ("Dequantize weights during matrix multiplication": the
 * weights stay int4; only their order changes). Writes into caller memory `dst` (device,
 * 256-byte aligned, at least moe_pack_bytes) and sets *packed (host) to a copy of *layer
 * whose w13_t, w13_tsb, w2_t, w2_tsb point into dst. The interchange arrays are only
 * read. Layout, for a matrix with R rows (2I for W13, H for W2) and reduction length K,
 * per expert, in blocks of 64 rows (W13 block j: gate rows 32j..32j+31, then up rows
 * 32j..32j+31; W2 block j: rows 64j..64j+63) and steps of 64 along K:
 *   *_t    uint8 [E+S][R/64][K/64][64 rows][32 bytes]  (the row's 32 code bytes of the step)
 *   *_tsb  bf16  [E+S][R/64][ceil(K/256)][64 rows][4 groups][scale, bias]  (zero padded)
 * and the router's two fp16 planes (router_planes).
 * Stream-ordered like every call; dst must not overlap the source arrays. */
moe_status moe_pack_weights(const moe_layer *layer, void *dst, size_t dst_bytes,
                            moe_layer *packed, void *stream);

/* Router, top-k and grouping: logits z = x W_r^T (+ b), k experts by (z desc, id asc),
 * weights = softmax restricted to the selection, then the per-expert histogram,
 * exclusive prefix scan and stable scatter ("Keep expert routing on the GPU").
 * x: [T, H] of act_dtype. All six moe_route_out buffers must be non-NULL. */
moe_status moe_route(const moe_layer *layer, const void *x, int64_t T,
                     const moe_route_out *out, void *ws, size_t ws_bytes, void *stream);

/* Whole layer for T >= 1 tokens (prefill path; "Optimizing On-Device Inference for Apple
 * Silicon", sections "Prefill: reuse weights and keep routing on the GPU", "Dequantize
 * weights during matrix multiplication" and "Match tile size to expert load"): routing as
 * moe_route, then for int4 (tiled weights required, see moe_pack_weights) a grouped
 * gate/up GEMM with SwiGLU, a grouped down GEMM (int4 codes dequantised to fp16 in
 * registers, fp16 MFMA, fp32 accumulation; the two in one persistent launch) and a weighted
 * combine back to token order. y[t] = shared(x_t) + sum_j w[t,j] expert_{ids[t,j]}(x_t)
 * (+ residual[t]). x, y, residual: [T, H] of act_dtype; residual may be NULL and may
 * alias y. route_out may be NULL; when given it receives the routing results.
 * Int4 calls with T * H * 2 >= 2^32 bytes run as consecutive calls of fewer tokens (the
 * same y); with route_out such a call returns MOE_E_UNSUPPORTED.
 * Results are deterministic: identical inputs give identical bytes. */
moe_status moe_prefill(const moe_layer *layer, const void *x, int64_t T, void *y,
                       const void *residual, const moe_route_out *route_out, void *ws,
                       size_t ws_bytes, void *stream);

/* One token (batch-1 decode path): router GEMV with top-k, then the 8+1 selected
 * experts' packed weights streamed through wavefront-reduced GEMVs on the vector ALUs
 * ("Optimize the one-row weight path", "Reduce intermediate and state traffic"):
 * gate/up + SwiGLU fused, then down + routing weights + shared expert fused.
 * x, y, residual: [1, H] of act_dtype; residual may be NULL and may alias y. */
moe_status moe_decode(const moe_layer *layer, const void *x, void *y, const void *residual,
                      void *ws, size_t ws_bytes, void *stream);

/* moe_decode for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels and results, with
 * the library's own scratch memory in place of a caller workspace. The scratch is one static
 * 4 MiB array per GPU that the library runs on, held from its first use on that GPU until
 * the process ends; a layer whose one-token workspace (moe_workspace_bytes with
 * max_tokens = 1) exceeds it is rejected with MOE_E_WORKSPACE before anything is enqueued.
 * The call allocates nothing and needs nothing cleared in the scratch. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two streams, two threads)
 * race and give undefined results; calls ordered on one stream are fine. Arguments as
 * moe_decode. */
moe_status moe_decode_noalloc(const moe_layer *layer, const void *x, void *y,
                              const void *residual, void *stream);

/* Ablations of the prefill path: the rejected designs of "Optimizing On-Device Inference
 * for Apple Silicon", section "Optimize sparse expert computation", rebuilt on the same
 * kernels so that each differs from the product path in one mechanism only. Every variant
 * computes exactly what moe_prefill computes for T > 8 (the grouped-GEMM path, which the
 * variants take for every T), so y is bit-identical to it:
 *   MOE_ABL_NONE              the grouped-GEMM path unchanged (the control)
 *   MOE_ABL_SEPARATE_DEQUANT  "Dequantize weights during matrix multiplication", its
 *       ablation: a separate pass expands the int4 weights of every expert that received
 *       rows (and the shared expert) into fp16 arrays in the workspace, and the GEMMs read
 *       those back instead of dequantising tiles on chip (as two launches, gate/up then
 *       down, instead of the persistent one)
 *   MOE_ABL_HOST_ROUTING      "Keep expert routing on the GPU", its ablation: the GPU stops
 *       after the router and top-k; the host reads the ids back, builds the histogram,
 *       offsets, per-block bases and tile map, uploads them and only then enqueues the
 *       scatter and the GEMMs. This variant synchronises `stream` twice and copies
 *       between host and device, unlike every other call, so it cannot be captured
 *   MOE_ABL_TILE_64           "Match tile size to expert load", its ablation: tiles of at
 *       most 64 rows, whatever the load
 *   MOE_ABL_FIXED_TILE        tiles of 128 rows of which every one multiplies all 128 rows'
 *       worth of blocks, however few rows it holds (no load adaptivity at all)
 *   MOE_ABL_TILE_128          tiles of at most 128 rows whatever the load (the per-call
 *       height choice off; each expert's last tile still only as high as its rows need)
 * Int4 layers only (MOE_E_UNSUPPORTED otherwise, and for T * H * 2 >= 2^32 bytes), tiled
 * weights required. Arguments as moe_prefill; the workspace must hold moe_ablation_workspace_bytes for the same variant
 * (for MOE_ABL_SEPARATE_DEQUANT that includes 2 bytes per expert weight). */
typedef enum {
  MOE_ABL_NONE = 0,
  MOE_ABL_SEPARATE_DEQUANT = 1,
  MOE_ABL_HOST_ROUTING = 2,
  MOE_ABL_TILE_64 = 3,
  MOE_ABL_FIXED_TILE = 4,
  MOE_ABL_TILE_128 = 5
} moe_ablation;

moe_status moe_ablation_workspace_bytes(const moe_layer *layer, int64_t max_tokens,
                                        int32_t variant, size_t *bytes);
moe_status moe_prefill_ablation(const moe_layer *layer, int32_t variant, const void *x, int64_t T,
                                void *y, const void *residual, void *ws, size_t ws_bytes,
                                void *stream);

/* Decode attention of one token over a grouped-query KV cache ("Optimizing On-Device
 * Inference for Apple Silicon", sections "Qwen creates three distinct workload shapes" and
 * "Read the attention cache efficiently"):
 *     out[h] = sum_t softmax_t(scale * q[h] . k[g, t]) v[g, t],   g = h / (n_q / n_kv)
 * over t = 0 .. ctx-1. The query heads sharing a KV head are packed into one workgroup,
 * which loads each cached row once for all of them; the cache is split into equal blocks
 * processed in parallel and merged (fp32 scores, softmax and sums).
 *   q    bf16 [n_q, head_dim]
 *   k, v bf16 caches: KV head g's row t at element g * kv_head_stride + t * head_dim
 *        (kv_head_stride >= ctx * head_dim, a multiple of 8)
 *   out  bf16 [n_q, head_dim]
 * Supported: head_dim == 256, n_q / n_kv in {1, 2, 4, 8}, 1 <= ctx <= 2^31. Pointers
 * 16-byte aligned; ws holds moe_attn_workspace_bytes(n_q, max_ctx >= ctx) bytes. */
moe_status moe_attn_workspace_bytes(int32_t n_q, int32_t n_kv, int32_t head_dim, int64_t max_ctx,
                                    size_t *bytes);
moe_status moe_attn_decode(const void *q, const void *k_cache, const void *v_cache, int32_t n_q,
                           int32_t n_kv, int32_t head_dim, int64_t ctx, int64_t kv_head_stride,
                           float scale, void *out, void *ws, size_t ws_bytes, void *stream);
/* The page's ablation of the packing: one workgroup per query head, so each cached row is
 * loaded once per query head ("Pack query heads to reuse KV rows"); the same blocks and the
 * same arithmetic per head, so out is bit-identical to moe_attn_decode. */
moe_status moe_attn_decode_unpacked(const void *q, const void *k_cache, const void *v_cache,
                                    int32_t n_q, int32_t n_kv, int32_t head_dim, int64_t ctx,
                                    int64_t kv_head_stride, float scale, void *out, void *ws,
                                    size_t ws_bytes, void *stream);

/* Gated DeltaNet recurrence over T tokens, state resident on chip for the whole scan
 * ("Optimizing On-Device Inference for Apple Silicon", sections "Qwen creates three distinct
 * workload shapes" and "Keep recurrent state on chip"), per value head j with key head
 * kh = j / (n_v / n_k):
 *     S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,   o_t = S_t q_t
 * (the gated delta rule; fp32 state and arithmetic, bf16 q, k, v, o).
 *   q, k   bf16 [T, n_k, d_k]        v  bf16 [T, n_v, d_v]
 *   alpha, beta  fp32 [T, n_v]       (gate and write strength of each token and head)
 *   state  fp32 [n_v, d_v, d_k]      S_0 on entry, overwritten with S_T (a prompt chunk
 *                                    continues from the previous chunk's state)
 *   out    bf16 [T, n_v, d_v]
 * Supported: d_k = d_v = 128, n_v a multiple of n_k, 0 <= T <= 2^24 (T = 0 leaves the state
 * as it is). Pointers 16-byte aligned (alpha and beta 4). No workspace. */
moe_status moe_gdn_scan(const void *q, const void *k, const void *v, const float *alpha,
                        const float *beta, int64_t T, int32_t n_k, int32_t n_v, int32_t d_k,
                        int32_t d_v, float *state, void *out, void *stream);

/* The same recurrence in its chunked form: tokens in chunks of 32; a first kernel forms, for
 * every chunk at once, the factors that depend on the inputs only (the WY factors of the
 * chunk's product of (I - beta k k^T) terms, the values they map to, the gate products and
 * the query-key products); a second walks the chunks in order with the state in registers,
 * so the sequential chain is T / 32 chunk steps instead of T token steps. Arguments as
 * moe_gdn_scan plus a workspace of moe_gdn_chunked_workspace_bytes (about 40 KB per value
 * head and chunk); results agree with moe_gdn_scan to fp32 rounding. */
moe_status moe_gdn_chunked_workspace_bytes(int64_t max_tokens, int32_t n_k, int32_t n_v,
                                           int32_t d_k, int32_t d_v, size_t *bytes);
moe_status moe_gdn_scan_chunked(const void *q, const void *k, const void *v, const float *alpha,
                                const float *beta, int64_t T, int32_t n_k, int32_t n_v,
                                int32_t d_k, int32_t d_v, float *state, void *out, void *ws,
                                size_t ws_bytes, void *stream);

/* Workspace bytes for moe_stack_forward with chunks of up to chunk_tokens rows. */
moe_status moe_stack_workspace_bytes(const moe_layer *layers, int32_t n_layers,
                                     int64_t chunk_tokens, size_t *bytes);

/* A stack of n_layers MoE layers (host array of descriptors) as pre-norm residual
 * blocks, applied in place to h [T, H]:
 *     for l = 0 .. n_layers-1:   h <- h + MoE_l(RMSNorm(h))
 * with RMSNorm of unit gain in fp64 arithmetic (eps as given), each normalised value
 * rounded once to the activation dtype (bf16: to nearest, ties to even) before the layer
 * reads it; router and experts read the same rounded row. Rows are processed in
 * chunks of at most chunk_tokens, each chunk through every layer, all reusing one
 * workspace of moe_stack_workspace_bytes ("Bound temporary memory with prompt chunking");
 * every layer is independent per token, so the chunk size does not change the result.
 * T == 1 runs the decode path of each layer, T > 1 the prefill path (int4 layers must be
 * packed). All layers need the same hidden size and activation dtype. */
moe_status moe_stack_forward(const moe_layer *layers, int32_t n_layers, void *h, int64_t T,
                             int64_t chunk_tokens, float eps, void *ws, size_t ws_bytes,
                             void *stream);

/* RMSNorm with unit gain for stacking layers: out[t] = h[t] / sqrt(mean(h[t]^2) + eps),
 * fp64 arithmetic, each value rounded once to act_dtype (bf16: to nearest, ties to even);
 * the normalisation moe_stack_forward applies. h, out: [T, H] of act_dtype (may alias). */
moe_status moe_rmsnorm(const void *h, int64_t T, int32_t hidden, float eps, int32_t act_dtype,
                       void *out, void *stream);

/* Measurement aids ("Optimizing On-Device Inference for Apple Silicon", section "Limits of
 * further optimization": kernels are judged against the fastest rate measured for their own
 * access pattern, besides the nominal peak). Neither computes anything of the layer.
 *
 * moe_decode_read_ceiling: the weight loads of one batch-1 decode kernel, from the same grid
 * and addresses, with the arithmetic taken out. part 0: the router GEMV's (router rows; the
 * router weights stand in for x); part 1: the gate/up kernel's (the experts ids[0..k-1], then
 * the shared expert); part 2: the down kernel's (the same experts). ids: device int32 [k];
 * sink: device uint32 [1], written only in the rare case a checksum equals a fixed word. The
 * layer must take the batch-1 fast path (packed, hidden 2048, intermediate 512); otherwise
 * MOE_E_UNSUPPORTED.
 *
 * moe_mfma_ceiling: a dense loop of v_mfma_f32_32x32x16_f16 on register operands over 512
 * workgroups of four waves (two per CU, like the grouped GEMMs), iters x 8 per wave; *flops
 * (host) receives the FLOP it executes. sink as above. The sustained rate depends on the
 * operands (the matrix cores draw power in proportion to the bits they switch, and the part
 * clocks down at its power limit): operands MOE_CEIL_FULL_MANTISSA runs on values with full
 * fp16 mantissas in (-1, 1), like a GEMM's activations and dequantised weights;
 * MOE_CEIL_LOW_ENTROPY on multiples of 1/2 below 4. Other values: MOE_E_INVALID. */
enum { MOE_CEIL_FULL_MANTISSA = 0, MOE_CEIL_LOW_ENTROPY = 1 };
moe_status moe_decode_read_ceiling(const moe_layer *layer, const int32_t *ids, int32_t part,
                                   uint32_t *sink, void *stream);
moe_status moe_mfma_ceiling(int32_t iters, int32_t operands, uint32_t *sink, double *flops,
                            void *stream);

/* Kernel timing for measurement tools. When enabled, every kernel the library launches
 * is dispatched with a start/stop HIP event pair bound to the dispatch itself
 * (hipExtLaunchKernel), on the kernel's stream. moe_profile_query() waits for the recorded
 * events, and returns the summed duration (ms) and launch count of every kernel whose
 * name equals `kernel`; moe_profile_reset() drops all records. Disabled by default. */
moe_status moe_profile_enable(int32_t on);
moe_status moe_profile_query(const char *kernel, double *total_ms, int64_t *launches);
moe_status moe_profile_reset(void);

#ifdef __cplusplus
}
#endif
#endif
