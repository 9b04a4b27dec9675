// moe_api.hip -- host side of the C ABI declared in include/moe.h: descriptor and
// size validation, the workspace plan, kernel dispatch and error reporting.
// No call allocates device memory, synchronises the host or copies device data to it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "moe.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status hip_fail(hipError_t e, const char *where) {
  return fail(MOE_E_HIP, "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxTokens = int64_t(1) << 24;

moe_status check_layer(const moe_layer *L) {
  if (!L) return fail(MOE_E_INVALID, "layer descriptor is NULL");
  if (L->abi_version != MOE_ABI_VERSION)
    return fail(MOE_E_INVALID, "abi_version %d, library is %d", L->abi_version,
                MOE_ABI_VERSION);
  if (L->hidden <= 0 || L->inter <= 0 || L->n_experts <= 0)
    return fail(MOE_E_INVALID, "hidden, inter and n_experts must be positive");
  if (L->top_k < 1 || L->top_k > L->n_experts)
    return fail(MOE_E_INVALID, "top_k %d outside [1, n_experts]", L->top_k);
  if (L->n_shared < 0 || L->n_shared > 1)
    return fail(MOE_E_INVALID, "n_shared must be 0 or 1");
  if (L->n_experts > moe::kMaxExperts)
    return fail(MOE_E_UNSUPPORTED, "n_experts %d > %d", L->n_experts, moe::kMaxExperts);
  if (L->top_k > moe::kMaxTopK)
    return fail(MOE_E_UNSUPPORTED, "top_k %d > %d", L->top_k, moe::kMaxTopK);
  if (L->hidden % 64 || L->inter % 64)
    return fail(MOE_E_UNSUPPORTED, "hidden and inter must be multiples of 64");
  if (!L->router_w || !L->w13_q || !L->w2_q)
    return fail(MOE_E_INVALID, "router_w, w13_q and w2_q must be non-NULL");
  if (L->w_format == MOE_W_INT4_G64) {
    if (L->act_dtype != MOE_ACT_BF16)
      return fail(MOE_E_UNSUPPORTED, "int4 weights need bf16 activations");
    if (L->hidden % 256 || L->inter % 128)
      return fail(MOE_E_UNSUPPORTED, "int4 layers need hidden %% 256 == 0 and inter %% 128 == 0");
    if (!L->w13_s || !L->w13_b || !L->w2_s || !L->w2_b)
      return fail(MOE_E_INVALID, "int4 scale/bias pointers must be non-NULL");
    if (!aligned16(L->w13_q) || !aligned16(L->w2_q) || ((uintptr_t)L->w13_s & 3) ||
        ((uintptr_t)L->w13_b & 3) || ((uintptr_t)L->w2_s & 3) || ((uintptr_t)L->w2_b & 3))
      return fail(MOE_E_INVALID,
                  "weight pointers misaligned (codes need 16 bytes, scales and biases 4)");
  } else if (L->w_format == MOE_W_F32) {
    if (L->act_dtype != MOE_ACT_F32)
      return fail(MOE_E_UNSUPPORTED, "fp32 weights need fp32 activations");
    if (!aligned16(L->w13_q) || !aligned16(L->w2_q))
      return fail(MOE_E_INVALID, "fp32 weight pointers must be 16-byte aligned");
  } else {
    return fail(MOE_E_INVALID, "unknown w_format %d", L->w_format);
  }
  if (!aligned16(L->router_w)) return fail(MOE_E_INVALID, "router_w must be 16-byte aligned");
  if (!aligned16(L->router_planes)) return fail(MOE_E_INVALID, "router_planes misaligned");
  if ((uintptr_t)L->router_b & 3) return fail(MOE_E_INVALID, "router_b misaligned");
  return MOE_OK;
}


// Workspace layout: the batch-1 decode buffers first, then the T-dependent region.
struct Plan {
  size_t dec_logits, dec_ids, dec_z, dec_h, dec_xn, st_z, st_ids, st_w, st_h;
  size_t logits, planes, ids, w, blk, chunk, offsets, sorted, slot, slot_w, x16, tiles, ntiles,
      h, out, sync;
  size_t total;
  int max_tiles;
};

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Tiles of r rows that k routed assignments per token plus the shared expert's T rows can
// need: every expert's rows in full tiles plus one partial tile.
size_t tile_bound(const moe_layer *L, size_t Tn, size_t r) {
  const size_t k = L->top_k, E = L->n_experts;
  return (k * Tn + r - 1) / r + E + (L->n_shared ? (Tn + r - 1) / r : 0);
}

// Tile-map entries for tile height 2^tile_shift, or (0) the height the scan picks from the
// load: 128 rows, or 64 / 32 rows only while the rows fill fewer than 4 * fill 32-row
// blocks, and then there are fewer tiles than blocks.
size_t max_tiles_for(const moe_layer *L, size_t Tn, int tile_shift) {
  if (tile_shift > 0) return tile_bound(L, Tn, (size_t)1 << tile_shift);
  const size_t small = std::min(tile_bound(L, Tn, 32), (size_t)4 * moe::gemm_fill(L->inter));
  return std::max(tile_bound(L, Tn, moe::kTileM), small);
}

Plan make_plan(const moe_layer *L, int64_t T, int tile_shift = 0) {
  Plan p{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t E = L->n_experts, k = L->top_k, S = L->n_shared, H = L->hidden, I = L->inter;
  const size_t Tn = (size_t)(T > 0 ? T : 1);
  const size_t NB = (Tn + moe::kRouteBlock - 1) / moe::kRouteBlock;
  p.dec_logits = take(E * 4);
  p.dec_ids = take(k * 4);
  p.dec_z = take(k * 4);
  p.dec_h = take((k + S) * I * 4);
  p.dec_xn = take(H * 2);
  // small-T path (2 .. kSmallT tokens)
  const size_t Ts = Tn < (size_t)moe::kSmallT ? Tn : (size_t)moe::kSmallT;
  p.st_z = take(Ts * E * 4);
  p.st_ids = take(Ts * k * 4);
  p.st_w = take(Ts * k * 4);
  p.st_h = take(Ts * (k + S) * I * 4);
  const size_t tiles = max_tiles_for(L, Tn, tile_shift);
  p.max_tiles = (int)tiles;
  const bool bf16 = L->act_dtype == MOE_ACT_BF16;
  p.logits = take((bf16 ? moe::kRouterParts : 1) * Tn * E * 4);
  p.planes = take(bf16 ? moe::router_frag_bytes((int)E, (int)H) : 0);
  p.ids = take(Tn * k * 4);
  p.w = take(Tn * k * 4);
  p.blk = take(NB * E * 4);
  p.offsets = take((E + 2) * 4);
  p.sorted = take(k * Tn * 4);
  p.slot = take(k * Tn * 4);
  p.tiles = take(tiles * 8);
  p.ntiles = take(4);
  if (L->w_format == MOE_W_INT4_G64) {
    p.slot_w = take(k * Tn * 4);
    p.x16 = take(Tn * H * 2);
    p.h = take((k + S) * Tn * I * 2);
    // the routed rows only: the shared expert's down projection adds them into y itself
    p.out = take(k * Tn * H * 2);
    p.sync = take(moe::sync_words(p.max_tiles) * 4);
  } else {
    p.h = take((k + S) * Tn * I * 4);
    p.slot_w = p.x16 = p.out = p.sync = off;
  }
  p.chunk = take((NB + moe::kChunkBlocks - 1) / moe::kChunkBlocks * E * 4);  // long calls
  p.total = off;
  return p;
}

template <typename Tp>
Tp *at(void *ws, size_t off) {
  return reinterpret_cast<Tp *>(static_cast<char *>(ws) + off);
}

moe::ExpertWeights weights_of(const moe_layer *L) {
  moe::ExpertWeights w{};
  if (L->w_format == MOE_W_INT4_G64) {
    w.w13_q = static_cast<const uint8_t *>(L->w13_q);
    w.w2_q = static_cast<const uint8_t *>(L->w2_q);
    w.w13_s = static_cast<const uint16_t *>(L->w13_s);
    w.w13_b = static_cast<const uint16_t *>(L->w13_b);
    w.w2_s = static_cast<const uint16_t *>(L->w2_s);
    w.w2_b = static_cast<const uint16_t *>(L->w2_b);
    w.w13_t = static_cast<const uint8_t *>(L->w13_t);
    w.w2_t = static_cast<const uint8_t *>(L->w2_t);
    w.w13_tsb = static_cast<const uint16_t *>(L->w13_tsb);
    w.w2_tsb = static_cast<const uint16_t *>(L->w2_tsb);
  } else {
    w.w13_f = static_cast<const float *>(L->w13_q);
    w.w2_f = static_cast<const float *>(L->w2_q);
  }
  return w;
}

// The grouped GEMMs read the tiled copy written by moe_pack_weights.
moe_status check_tiled(const moe_layer *L) {
  if (!L->w13_t || !L->w13_tsb || !L->w2_t || !L->w2_tsb)
    return fail(MOE_E_INVALID, "int4 prefill needs the tiled weights (call moe_pack_weights)");
  if (!aligned16(L->w13_t) || !aligned16(L->w13_tsb) || !aligned16(L->w2_t) ||
      !aligned16(L->w2_tsb))
    return fail(MOE_E_INVALID, "tiled weight pointers must be 16-byte aligned");
  return MOE_OK;
}

struct PackPlan {
  size_t w13_t, w13_tsb, w2_t, w2_tsb, planes, total;
};

PackPlan pack_plan(const moe_layer *L) {
  const int n = L->n_experts + L->n_shared, H = L->hidden, I = L->inter;
  PackPlan p{};
  size_t off = 0;
  p.w13_t = off;
  off += align256(moe::tiled_code_bytes(n, 2 * I, H));
  p.w13_tsb = off;
  off += align256(moe::tiled_sb_bytes(n, 2 * I, H));
  p.w2_t = off;
  off += align256(moe::tiled_code_bytes(n, H, I));
  p.w2_tsb = off;
  off += align256(moe::tiled_sb_bytes(n, H, I));
  p.planes = off;
  off += align256(moe::router_frag_bytes(L->n_experts, H));
  p.total = off;
  return p;
}

struct StackPlan {
  size_t norm, layer_ws, total;
};

// Workspace of a stack: the normalised rows of one chunk, then one layer workspace (sized
// for the largest layer) that every layer and chunk reuses.
moe_status stack_plan(const moe_layer *layers, int32_t n_layers, int64_t chunk, StackPlan *sp) {
  if (!layers || n_layers < 1) return fail(MOE_E_INVALID, "need at least one layer");
  if (chunk < 1 || chunk > kMaxTokens) return fail(MOE_E_INVALID, "bad chunk_tokens");
  size_t lws = 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    const moe_status st = check_layer(&layers[l]);
    if (st) return st;
    if (layers[l].hidden != layers[0].hidden || layers[l].act_dtype != layers[0].act_dtype)
      return fail(MOE_E_INVALID, "layer %d: hidden size or activation dtype differs", l);
    lws = std::max(lws, make_plan(&layers[l], chunk).total);
  }
  const size_t elt = layers[0].act_dtype == MOE_ACT_BF16 ? 2 : 4;
  sp->norm = 0;
  sp->layer_ws = align256((size_t)chunk * layers[0].hidden * elt);
  sp->total = sp->layer_ws + lws;
  return MOE_OK;
}

moe_status check_ws(const moe_layer *L, int64_t T, void *ws, size_t ws_bytes, Plan *p) {
  *p = make_plan(L, T);
  if (!ws) return fail(MOE_E_INVALID, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_E_INVALID, "workspace must be 16-byte aligned");
  if (ws_bytes < p->total)
    return fail(MOE_E_WORKSPACE, "workspace %zu bytes < %zu needed for T=%lld", ws_bytes,
                p->total, (long long)T);
  return MOE_OK;
}

moe::RouteArgs route_args(const moe_layer *L, const void *x, int64_t T) {
  moe::RouteArgs a{};
  a.bf16 = L->act_dtype == MOE_ACT_BF16;
  a.x = x;
  a.router_w = L->router_w;
  a.router_b = L->router_b;
  a.T = T;
  a.H = L->hidden;
  a.E = L->n_experts;
  a.k = L->top_k;
  a.S = L->n_shared;
  a.I = L->inter;
  if (a.bf16 && L->router_planes) {
    a.router_planes = const_cast<uint16_t *>(static_cast<const uint16_t *>(L->router_planes));
    a.planes_ready = true;
  }
  return a;
}

// Routing results go to the caller's buffers when given, else to the workspace.
void route_targets(moe::RouteArgs &a, const Plan &p, void *ws, const moe_route_out *ro) {
  a.logits = at<float>(ws, p.logits);
  if (!a.planes_ready) a.router_planes = at<uint16_t>(ws, p.planes);
  a.blk = at<int32_t>(ws, p.blk);
  a.chunk = (a.T + moe::kRouteBlock - 1) / moe::kRouteBlock > moe::kChunkFromBlocks
                ? at<int32_t>(ws, p.chunk)
                : nullptr;
  a.offsets = at<int32_t>(ws, p.offsets);
  a.tiles = at<int2>(ws, p.tiles);
  a.n_tiles = at<int32_t>(ws, p.ntiles);
  a.ids = ro ? ro->topk_ids : at<int32_t>(ws, p.ids);
  a.w = ro ? ro->topk_w : at<float>(ws, p.w);
  a.sorted_tok = ro ? ro->sorted_tok : at<int32_t>(ws, p.sorted);
  a.slot_of = ro ? ro->slot_of : at<int32_t>(ws, p.slot);
  a.counts_user = ro ? ro->counts : nullptr;
  a.offsets_user = ro ? ro->offsets : nullptr;
  a.slot_w = nullptr;
  a.x16 = nullptr;
}

moe_status check_route_out(const moe_route_out *ro) {
  if (!ro->topk_ids || !ro->topk_w || !ro->counts || !ro->offsets || !ro->sorted_tok ||
      !ro->slot_of)
    return fail(MOE_E_INVALID, "every moe_route_out buffer must be non-NULL");
  return MOE_OK;
}

// ---- kernel timing -----------------------------------------------------------------------
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;
std::atomic<bool> g_prof_on{false};

}  // namespace

namespace moe {

bool prof_events(const char *name, hipEvent_t *start, hipEvent_t *stop) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return false;
  ProfRec r{name, nullptr, nullptr};
  if (hipEventCreate(&r.a) != hipSuccess) return false;
  if (hipEventCreate(&r.b) != hipSuccess) {
    (void)hipEventDestroy(r.a);
    return false;
  }
  *start = r.a;
  *stop = r.b;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back(r);
  return true;
}

}  // namespace moe

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_last_error(void) { return g_err.c_str(); }

moe_status moe_workspace_bytes(const moe_layer *layer, int64_t max_tokens, size_t *bytes) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (!bytes) return fail(MOE_E_INVALID, "bytes is NULL");
  if (max_tokens < 1 || max_tokens > kMaxTokens)
    return fail(MOE_E_INVALID, "max_tokens %lld outside [1, %lld]", (long long)max_tokens,
                (long long)kMaxTokens);
  *bytes = make_plan(layer, max_tokens).total;
  return MOE_OK;
}

moe_status moe_pack_bytes(const moe_layer *layer, size_t *bytes) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (!bytes) return fail(MOE_E_INVALID, "bytes is NULL");
  if (layer->w_format != MOE_W_INT4_G64)
    return fail(MOE_E_UNSUPPORTED, "only int4 layers are packed");
  *bytes = pack_plan(layer).total;
  return MOE_OK;
}

moe_status moe_pack_weights(const moe_layer *layer, void *dst, size_t dst_bytes,
                            moe_layer *packed, void *stream) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (layer->w_format != MOE_W_INT4_G64)
    return fail(MOE_E_UNSUPPORTED, "only int4 layers are packed");
  if (!packed) return fail(MOE_E_INVALID, "packed is NULL");
  if (!dst || (reinterpret_cast<uintptr_t>(dst) & 255u))
    return fail(MOE_E_INVALID, "dst must be non-NULL and 256-byte aligned");
  const PackPlan pp = pack_plan(layer);
  if (dst_bytes < pp.total)
    return fail(MOE_E_WORKSPACE, "dst holds %zu bytes, packing needs %zu", dst_bytes, pp.total);
  const int n = layer->n_experts + layer->n_shared;
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::PackArgs a{};
  a.n_mat = n;
  a.inter = layer->inter;
  a.gate_up = true;
  a.rows = 2 * layer->inter;
  a.K = layer->hidden;
  a.q = static_cast<const uint8_t *>(layer->w13_q);
  a.sc = static_cast<const uint16_t *>(layer->w13_s);
  a.bi = static_cast<const uint16_t *>(layer->w13_b);
  a.t = at<uint8_t>(dst, pp.w13_t);
  a.tsb = at<uint16_t>(dst, pp.w13_tsb);
  hipError_t e = moe::launch_pack(a, s);
  if (e != hipSuccess) return hip_fail(e, "moe_pack_weights gate/up");
  a.gate_up = false;
  a.rows = layer->hidden;
  a.K = layer->inter;
  a.q = static_cast<const uint8_t *>(layer->w2_q);
  a.sc = static_cast<const uint16_t *>(layer->w2_s);
  a.bi = static_cast<const uint16_t *>(layer->w2_b);
  a.t = at<uint8_t>(dst, pp.w2_t);
  a.tsb = at<uint16_t>(dst, pp.w2_tsb);
  if ((e = moe::launch_pack(a, s)) != hipSuccess) return hip_fail(e, "moe_pack_weights down");
  if ((e = moe::launch_router_split(layer->router_w, layer->n_experts, layer->hidden,
                                    at<uint16_t>(dst, pp.planes), s)) != hipSuccess)
    return hip_fail(e, "moe_pack_weights router");
  *packed = *layer;
  packed->w13_t = at<uint8_t>(dst, pp.w13_t);
  packed->w13_tsb = at<uint16_t>(dst, pp.w13_tsb);
  packed->w2_t = at<uint8_t>(dst, pp.w2_t);
  packed->w2_tsb = at<uint16_t>(dst, pp.w2_tsb);
  packed->router_planes = at<uint16_t>(dst, pp.planes);
  return MOE_OK;
}

moe_status moe_route(const moe_layer *layer, const void *x, int64_t T, const moe_route_out *out,
                     void *ws, size_t ws_bytes, void *stream) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (T < 0 || T > kMaxTokens) return fail(MOE_E_INVALID, "T %lld out of range", (long long)T);
  if (!out) return fail(MOE_E_INVALID, "route output descriptor is NULL");
  if ((st = check_route_out(out))) return st;
  if (!x || !aligned16(x)) return fail(MOE_E_INVALID, "x must be non-NULL and 16-byte aligned");
  Plan p;
  if ((st = check_ws(layer, T, ws, ws_bytes, &p))) return st;
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::RouteArgs ra = route_args(layer, x, T);
  route_targets(ra, p, ws, out);
  hipError_t e = moe::launch_route_prefill(ra, s);
  if (e != hipSuccess) return hip_fail(e, "moe_route");
  return MOE_OK;
}

// Work queues of the fused gate/up + down launch: one per XCD of the current device (32 CUs
// each), or 0 where the count is not a power of two up to kMaxQueues (then the two GEMMs run
// as separate launches).
static int device_queues() {
  static std::atomic<int> cache[64];  // queues + 1 per device id, 0 = not yet known
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    const int x = cus % 32 == 0 ? cus / 32 : 0;
    c = 1 + ((x >= 1 && x <= moe::kMaxQueues && (x & (x - 1)) == 0) ? x : 0);
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c - 1;
}

// Grouped GEMMs of an int4 layer over the routing in ra (tables already on the device).
static moe::GroupedArgs grouped_args(const moe_layer *layer, const moe::RouteArgs &ra, void *ws,
                                     const Plan &p) {
  moe::GroupedArgs ga{};
  ga.x16 = ra.x16;
  ga.sorted_tok = ra.sorted_tok;
  ga.slot_w = ra.slot_w;
  ga.offsets = ra.offsets;
  ga.tiles = ra.tiles;
  ga.n_tiles = ra.n_tiles;
  ga.max_tiles = p.max_tiles;
  ga.T = ra.T;
  ga.H = layer->hidden;
  ga.I = layer->inter;
  ga.E = layer->n_experts;
  ga.k = layer->top_k;
  ga.S = layer->n_shared;
  ga.wt = weights_of(layer);
  ga.h16 = at<uint16_t>(ws, p.h);
  ga.out = at<uint16_t>(ws, p.out);
  // the fused launch needs the queue words zeroed by this call's k_group (ra.sync)
  ga.n_queues = ra.sync ? device_queues() : 0;
  ga.sync = ga.n_queues ? ra.sync : nullptr;
  return ga;
}

// gate/up GEMM, down GEMM and the weighted combine into y
static moe_status run_grouped(const moe_layer *layer, const moe::GroupedArgs &ga,
                              const moe::RouteArgs &ra, const void *residual, void *y,
                              hipStream_t s) {
  hipError_t e;
  moe::GroupedArgs gd = ga;
  if (layer->n_shared) {
    // the routed experts' down projection skips the shared expert, whose down projection
    // runs afterwards with the combine fused
    gd.fused_combine = 1;
    gd.slot_of = ra.slot_of;
    gd.residual = static_cast<const uint16_t *>(residual);
    gd.y = static_cast<uint16_t *>(y);
  }
  if (gd.sync && !gd.w13_x) {
    // gate/up and down in one persistent launch
    if ((e = moe::launch_grouped_fused(gd, s)) != hipSuccess)
      return hip_fail(e, "moe_prefill gate/up + down");
  } else {
    if ((e = moe::launch_grouped_gateup(ga, s)) != hipSuccess)
      return hip_fail(e, "moe_prefill gate/up");
    if ((e = moe::launch_grouped_down(gd, s)) != hipSuccess)
      return hip_fail(e, "moe_prefill down");
  }
  if (layer->n_shared) {
    if ((e = moe::launch_shared_down_combine(gd, s)) != hipSuccess)
      return hip_fail(e, "moe_prefill shared down + combine");
    return MOE_OK;
  }
  moe::CombineArgs ca{};
  ca.out = ga.out;
  ca.slot_of = ra.slot_of;
  ca.residual = static_cast<const uint16_t *>(residual);
  ca.y = static_cast<uint16_t *>(y);
  ca.T = ra.T;
  ca.H = layer->hidden;
  ca.k = layer->top_k;
  if ((e = moe::launch_combine(ca, s)) != hipSuccess) return hip_fail(e, "moe_prefill combine");
  return MOE_OK;
}

// The layer for T >= 1 tokens after validation; p is the workspace plan for T tokens.
static bool decode_fast(const moe_layer *layer);

static moe_status prefill_impl(const moe_layer *layer, const void *x, int64_t T, void *y,
                               const void *residual, const moe_route_out *route_out, void *ws,
                               const Plan &p, hipStream_t s) {
  if (!route_out && T <= moe::kSmallT && decode_fast(layer)) {
    // a few tokens: the decode kernels' three-kernel structure, weights read once per
    // selected expert (no routing tables, tile map or grouped GEMMs)
    moe::DecodeArgs da{};
    da.x = static_cast<const uint16_t *>(x);
    da.router_w = layer->router_w;
    da.router_b = layer->router_b;
    da.wt = weights_of(layer);
    da.residual = static_cast<const uint16_t *>(residual);
    da.y = static_cast<uint16_t *>(y);
    da.z = at<float>(ws, p.st_z);
    da.h = at<float>(ws, p.st_h);
    da.sel_ids = at<int32_t>(ws, p.st_ids);
    da.sel_z = at<float>(ws, p.st_w);
    da.sel_is_w = 1;
    da.T = (int)T;
    da.H = layer->hidden;
    da.I = layer->inter;
    da.E = layer->n_experts;
    da.k = layer->top_k;
    da.S = layer->n_shared;
    const hipError_t e = moe::launch_small_t(da, s);
    if (e != hipSuccess) return hip_fail(e, "moe_prefill (small T)");
    return MOE_OK;
  }
  const bool int4 = layer->w_format == MOE_W_INT4_G64;
  // The grouped GEMMs address gathered x rows by 32-bit byte offsets: T * H * 2 < 2^32.
  // Larger calls run as consecutive calls of fewer tokens (every token's result is the same).
  const int64_t t_max = (int64_t)(0xFFFFFFFFull / (2ull * (uint64_t)layer->hidden)) & ~int64_t(63);
  if (int4 && T > t_max) {
    if (route_out)
      return fail(MOE_E_UNSUPPORTED, "route_out needs T * hidden * 2 < 2^32 (T = %lld)",
                  (long long)T);
    const bool bf16 = layer->act_dtype == MOE_ACT_BF16;
    const size_t row = (size_t)layer->hidden * (bf16 ? 2 : 4), yrow = row;  // x, y, residual
    for (int64_t r0 = 0; r0 < T; r0 += t_max) {
      const int64_t n = std::min(t_max, T - r0);
      const moe_status st = prefill_impl(
          layer, static_cast<const char *>(x) + r0 * row, n,
          static_cast<char *>(y) + r0 * yrow,
          residual ? static_cast<const char *>(residual) + r0 * yrow : nullptr, nullptr, ws, p,
          s);
      if (st) return st;
    }
    return MOE_OK;
  }
  moe::RouteArgs ra = route_args(layer, x, T);
  route_targets(ra, p, ws, route_out);
  if (int4) {
    ra.slot_w = at<float>(ws, p.slot_w);
    ra.x16 = at<uint16_t>(ws, p.x16);
    ra.sync = at<int32_t>(ws, p.sync);
    ra.n_sync = (int)moe::sync_words(p.max_tiles);
  }
  hipError_t e = moe::launch_route_prefill(ra, s);
  if (e != hipSuccess) return hip_fail(e, "moe_prefill route");
  const moe::ExpertWeights wt = weights_of(layer);
  if (int4) {
    moe::GroupedArgs ga = grouped_args(layer, ra, ws, p);
    return run_grouped(layer, ga, ra, residual, y, s);
  } else {
    moe::TokenArgs ta{};
    ta.bf16 = false;
    ta.int4 = false;
    ta.x = x;
    ta.ids = ra.ids;
    ta.w = ra.w;
    ta.residual = residual;
    ta.y = y;
    ta.h = at<float>(ws, p.h);
    ta.T = T;
    ta.H = layer->hidden;
    ta.I = layer->inter;
    ta.E = layer->n_experts;
    ta.k = layer->top_k;
    ta.S = layer->n_shared;
    ta.wt = wt;
    if ((e = moe::launch_token_experts(ta, s)) != hipSuccess)
      return hip_fail(e, "moe_prefill experts");
  }
  return MOE_OK;
}

moe_status moe_prefill(const moe_layer *layer, const void *x, int64_t T, void *y,
                       const void *residual, const moe_route_out *route_out, void *ws,
                       size_t ws_bytes, void *stream) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (T < 0 || T > kMaxTokens) return fail(MOE_E_INVALID, "T %lld out of range", (long long)T);
  if (T == 0) return MOE_OK;  // empty input: nothing to read or write
  if (!x || !y || !aligned16(x) || !aligned16(y))
    return fail(MOE_E_INVALID, "x and y must be non-NULL and 16-byte aligned");
  if (residual && !aligned16(residual)) return fail(MOE_E_INVALID, "residual misaligned");
  if (route_out && (st = check_route_out(route_out))) return st;
  if (layer->w_format == MOE_W_INT4_G64 && (st = check_tiled(layer))) return st;
  Plan p;
  if ((st = check_ws(layer, T, ws, ws_bytes, &p))) return st;
  return prefill_impl(layer, x, T, y, residual, route_out, ws, p, static_cast<hipStream_t>(stream));
}

// ---- ablations of the prefill path ------------------------------------------------------
namespace {

// Tile height of a variant: fixed (log2 rows) or 0, the product's choice from the load.
int abl_shift(int variant) {
  switch (variant) {
    case MOE_ABL_TILE_64: return 6;
    case MOE_ABL_TILE_128:
    case MOE_ABL_FIXED_TILE: return 7;
    default: return 0;
  }
}

// Workspace of moe_prefill_ablation: a prefill plan sized for the variant's tiles, one
// contiguous block of routing tables the host can upload in one copy, and (separate
// dequantisation) the expanded fp16 weights.
struct AblPlan {
  Plan p;
  size_t tab, tab_bytes, x13, x2, total;
  size_t tab_offsets, tab_ntiles, tab_tiles, tab_blk;  // int32 word offsets inside tab
};

AblPlan abl_plan(const moe_layer *L, int64_t T, int variant) {
  AblPlan a{};
  a.p = make_plan(L, T, abl_shift(variant));
  const size_t E = L->n_experts, Tn = (size_t)(T > 0 ? T : 1);
  const size_t NB = (Tn + moe::kRouteBlock - 1) / moe::kRouteBlock;
  a.tab_offsets = 0;
  a.tab_ntiles = E + 2;
  a.tab_tiles = (E + 3 + 1) & ~size_t(1);  // int2 entries start on an even word
  a.tab_blk = a.tab_tiles + 2 * (size_t)a.p.max_tiles;
  a.tab_bytes = (a.tab_blk + NB * E) * 4;
  size_t off = a.p.total;
  a.tab = off;
  off += align256(a.tab_bytes);
  a.x13 = a.x2 = off;
  if (variant == MOE_ABL_SEPARATE_DEQUANT) {
    const int n = L->n_experts + L->n_shared;
    a.x13 = off;
    off += align256(moe::expanded_bytes(n, 2 * L->inter, L->hidden));
    a.x2 = off;
    off += align256(moe::expanded_bytes(n, L->hidden, L->inter));
  }
  a.total = off;
  return a;
}

// Host copy of the device scan (group_tables): per-block bases, offsets, the tile height (fixed
// or chosen from the load by the same rule) and the tile map in the same order and
// encoding (full tiles, the shared expert's full tiles, partial tiles by height, the
// shared expert's partial tile), from the top-k ids read back from the device.
int host_tables(const std::vector<int32_t> &ids, int64_t T, int E, int k, int S, int I,
                int tile_shift, const AblPlan &ap, std::vector<int32_t> &tab) {
  const int64_t NB = (T + moe::kRouteBlock - 1) / moe::kRouteBlock;
  tab.assign(ap.tab_bytes / 4, 0);
  int32_t *blk = tab.data() + ap.tab_blk;
  std::vector<int64_t> run(E, 0);
  for (int64_t b = 0; b < NB; ++b) {
    int32_t *row = blk + b * E;
    for (int e = 0; e < E; ++e) row[e] = (int32_t)run[e];
    const int64_t t1 = std::min<int64_t>(T, (b + 1) * moe::kRouteBlock);
    for (int64_t i = b * moe::kRouteBlock * k; i < t1 * k; ++i) {
      if (ids[i] < 0 || ids[i] >= E) return -1;
      ++run[ids[i]];
    }
  }
  int32_t *off = tab.data() + ap.tab_offsets;
  int64_t acc = 0;
  for (int e = 0; e < E; ++e) {
    off[e] = (int32_t)acc;
    acc += run[e];
  }
  off[E] = (int32_t)acc;
  off[E + 1] = (int32_t)(acc + (S ? T : 0));
  const bool chosen = tile_shift <= 0;
  if (chosen) {
    int64_t nblk = S ? (T + 31) / 32 : 0;
    for (int e = 0; e < E; ++e) nblk += (run[e] + 31) / 32;
    const int fill = moe::gemm_fill(I);
    tile_shift = nblk >= 4 * fill ? 7 : nblk >= 2 * fill ? 6 : 5;
  }
  const int64_t tr = int64_t(1) << tile_shift;
  // a group's remainder rows: those left to a partial tile (0 when they joined the last
  // full tile, which 128-row tiles chosen from the load do for 1..32 rows)
  const bool merge = chosen && tile_shift == 7;
  auto rem_of = [&](int64_t rows) {
    const int64_t r = rows % tr;
    return merge && rows >= tr && r <= 32 ? 0 : r;
  };
  int2 *tiles = reinterpret_cast<int2 *>(tab.data() + ap.tab_tiles);
  auto tile = [](int g, int64_t rows, int64_t r0) { return make_int2(g | (int)rows << 16, (int)r0); };
  int n_out = 0;
  auto full_tiles = [&](int g, int64_t rows) {
    const int64_t nf = rows / tr, extra = rows % tr - rem_of(rows);
    for (int64_t i = 0; i < nf; ++i) tiles[n_out++] = tile(g, i + 1 < nf ? tr : tr + extra, i * tr);
  };
  for (int e = 0; e < E; ++e) full_tiles(e, run[e]);
  if (S) full_tiles(E, T);
  for (int mb = 4; mb >= 1; --mb)
    for (int e = 0; e < E; ++e) {
      const int64_t rem = rem_of(run[e]);
      if (rem && (rem + 31) / 32 == mb) tiles[n_out++] = tile(e, rem, run[e] - rem);
    }
  if (S && rem_of(T)) tiles[n_out++] = tile(E, rem_of(T), T - rem_of(T));
  const int n = n_out;
  tab[ap.tab_ntiles] = n;
  return n;
}

}  // namespace

moe_status moe_ablation_workspace_bytes(const moe_layer *layer, int64_t max_tokens,
                                        int32_t variant, size_t *bytes) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (!bytes) return fail(MOE_E_INVALID, "bytes is NULL");
  if (variant < MOE_ABL_NONE || variant > MOE_ABL_TILE_128)
    return fail(MOE_E_INVALID, "unknown ablation %d", variant);
  if (max_tokens < 0 || max_tokens > kMaxTokens)
    return fail(MOE_E_INVALID, "max_tokens %lld out of range", (long long)max_tokens);
  *bytes = abl_plan(layer, max_tokens, variant).total;
  return MOE_OK;
}

moe_status moe_prefill_ablation(const moe_layer *layer, int32_t variant, const void *x, int64_t T,
                                void *y, const void *residual, void *ws, size_t ws_bytes,
                                void *stream) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (variant < MOE_ABL_NONE || variant > MOE_ABL_TILE_128)
    return fail(MOE_E_INVALID, "unknown ablation %d", variant);
  if (layer->w_format != MOE_W_INT4_G64)
    return fail(MOE_E_UNSUPPORTED, "ablations cover the int4 grouped-GEMM path only");
  if (T < 0 || T > kMaxTokens) return fail(MOE_E_INVALID, "T %lld out of range", (long long)T);
  if (T == 0) return MOE_OK;
  if ((uint64_t)T * 2 * (uint64_t)layer->hidden > 0xFFFFFFFFull)
    return fail(MOE_E_UNSUPPORTED, "ablations need T * hidden * 2 < 2^32 (T = %lld)", (long long)T);
  if (!x || !y || !aligned16(x) || !aligned16(y))
    return fail(MOE_E_INVALID, "x and y must be non-NULL and 16-byte aligned");
  if (residual && !aligned16(residual)) return fail(MOE_E_INVALID, "residual misaligned");
  if ((st = check_tiled(layer))) return st;
  const AblPlan ap = abl_plan(layer, T, variant);
  if (!ws || !aligned16(ws)) return fail(MOE_E_INVALID, "workspace NULL or misaligned");
  if (ws_bytes < ap.total)
    return fail(MOE_E_WORKSPACE, "workspace %zu bytes < %zu needed for T=%lld, ablation %d",
                ws_bytes, ap.total, (long long)T, variant);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Plan &p = ap.p;
  moe::RouteArgs ra = route_args(layer, x, T);
  route_targets(ra, p, ws, nullptr);
  ra.slot_w = at<float>(ws, p.slot_w);
  ra.x16 = at<uint16_t>(ws, p.x16);
  ra.tile_shift = abl_shift(variant);
  // the persistent gate/up + down launch as in moe_prefill, except with the separate
  // dequantisation pass (its expanded-weight GEMMs run as two launches)
  if (variant != MOE_ABL_SEPARATE_DEQUANT) {
    ra.sync = at<int32_t>(ws, p.sync);
    ra.n_sync = (int)moe::sync_words(p.max_tiles);
  }
  hipError_t e;
  int host_tiles = -1;
  if (variant == MOE_ABL_HOST_ROUTING) {
    // the GPU stops after top-k; the host reads the ids, builds the tables and uploads them
    if ((e = moe::launch_route_topk(ra, s)) != hipSuccess) return hip_fail(e, "ablation route");
    std::vector<int32_t> ids((size_t)T * layer->top_k), tab;
    if ((e = hipMemcpyAsync(ids.data(), ra.ids, ids.size() * 4, hipMemcpyDeviceToHost, s)) ||
        (e = hipStreamSynchronize(s)))
      return hip_fail(e, "ablation: reading the top-k ids");
    host_tiles = host_tables(ids, T, layer->n_experts, layer->top_k, layer->n_shared,
                             layer->inter, ra.tile_shift, ap, tab);
    if (host_tiles < 0) return fail(MOE_E_HIP, "ablation: top-k ids out of range");
    int32_t *dtab = at<int32_t>(ws, ap.tab);
    if ((e = hipMemcpyAsync(dtab, tab.data(), ap.tab_bytes, hipMemcpyHostToDevice, s)) ||
        (e = hipStreamSynchronize(s)))  // tab is host memory local to this call
      return hip_fail(e, "ablation: uploading the routing tables");
    // the queue words k_group would have zeroed
    const std::vector<int32_t> zeros((size_t)ra.n_sync, 0);
    if ((e = hipMemcpyAsync(ra.sync, zeros.data(), zeros.size() * 4, hipMemcpyHostToDevice, s)) ||
        (e = hipStreamSynchronize(s)))
      return hip_fail(e, "ablation: clearing the work-queue words");
    ra.offsets = dtab + ap.tab_offsets;
    ra.n_tiles = dtab + ap.tab_ntiles;
    ra.tiles = reinterpret_cast<int2 *>(dtab + ap.tab_tiles);
    ra.blk = dtab + ap.tab_blk;
    if ((e = moe::launch_route_scatter(ra, s)) != hipSuccess)
      return hip_fail(e, "ablation scatter");
  } else if ((e = moe::launch_route_prefill(ra, s)) != hipSuccess) {
    return hip_fail(e, "ablation route");
  }
  moe::GroupedArgs ga = grouped_args(layer, ra, ws, p);
  // grid: the bound for the variant's tile heights, or exactly the tiles the host listed
  if (host_tiles >= 0) ga.max_tiles = host_tiles;
  ga.fixed_mb = variant == MOE_ABL_FIXED_TILE;
  if (variant == MOE_ABL_SEPARATE_DEQUANT) {
    ga.w13_x = at<uint16_t>(ws, ap.x13);
    ga.w2_x = at<uint16_t>(ws, ap.x2);
    if ((e = moe::launch_expand(ga, s)) != hipSuccess) return hip_fail(e, "ablation dequant pass");
  }
  return run_grouped(layer, ga, ra, residual, y, s);
}

// One token after validation; p is a workspace plan for at least one token.
static bool decode_fast(const moe_layer *layer) {
  return moe::decode_gemv_supported(layer->hidden, layer->inter, layer->n_experts,
                                    layer->top_k, layer->n_shared,
                                    layer->w_format == MOE_W_INT4_G64) &&
         layer->w13_t && layer->w13_tsb && layer->w2_t && layer->w2_tsb;
}

// One token after validation; p is a workspace plan for at least one token. norm_eps >= 0
// (three-kernel path only) makes the layer read RMSNorm(x) instead of x.
static moe_status decode_impl(const moe_layer *layer, const void *x, void *y,
                              const void *residual, void *ws, const Plan &p, hipStream_t s,
                              float norm_eps = -1.0f) {
  hipError_t e;
  const bool int4 = layer->w_format == MOE_W_INT4_G64;
  // the three-kernel path reads the tiled weights; unpacked layers take the generic path
  if (decode_fast(layer)) {
    moe::DecodeArgs da{};
    da.x = static_cast<const uint16_t *>(x);
    da.router_w = layer->router_w;
    da.router_b = layer->router_b;
    da.wt = weights_of(layer);
    da.residual = static_cast<const uint16_t *>(residual);
    da.y = static_cast<uint16_t *>(y);
    da.z = at<float>(ws, p.dec_logits);
    da.h = at<float>(ws, p.dec_h);
    da.sel_ids = at<int32_t>(ws, p.dec_ids);
    da.sel_z = at<float>(ws, p.dec_z);
    da.H = layer->hidden;
    da.I = layer->inter;
    da.E = layer->n_experts;
    da.k = layer->top_k;
    da.S = layer->n_shared;
    da.T = 1;
    da.norm = norm_eps >= 0.f;
    da.eps = norm_eps;
    da.xn = at<uint16_t>(ws, p.dec_xn);
    if ((e = moe::launch_decode_gemv(da, s)) != hipSuccess) return hip_fail(e, "moe_decode");
    return MOE_OK;
  }
  // other shapes: the T = 1 case of the routing kernels, then the per-token GEMVs
  moe::RouteArgs ra = route_args(layer, x, 1);
  route_targets(ra, p, ws, nullptr);
  if ((e = moe::launch_route_prefill(ra, s)) != hipSuccess) return hip_fail(e, "moe_decode route");
  moe::TokenArgs ta{};
  ta.bf16 = layer->act_dtype == MOE_ACT_BF16;
  ta.int4 = int4;
  ta.x = x;
  ta.ids = ra.ids;
  ta.w = ra.w;
  ta.residual = residual;
  ta.y = y;
  ta.h = at<float>(ws, p.dec_h);
  ta.T = 1;
  ta.H = layer->hidden;
  ta.I = layer->inter;
  ta.E = layer->n_experts;
  ta.k = layer->top_k;
  ta.S = layer->n_shared;
  ta.wt = weights_of(layer);
  if ((e = moe::launch_token_experts(ta, s)) != hipSuccess)
    return hip_fail(e, "moe_decode experts");
  return MOE_OK;
}

moe_status moe_decode(const moe_layer *layer, const void *x, void *y, const void *residual,
                      void *ws, size_t ws_bytes, void *stream) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (!x || !y || !aligned16(x) || !aligned16(y))
    return fail(MOE_E_INVALID, "x and y must be non-NULL and 16-byte aligned");
  if (residual && !aligned16(residual)) return fail(MOE_E_INVALID, "residual misaligned");
  Plan p;
  if ((st = check_ws(layer, 1, ws, ws_bytes, &p))) return st;
  return decode_impl(layer, x, y, residual, ws, p, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- decode without a caller workspace ------------------------------------------------------
// Scratch memory of moe_decode_noalloc: one array per GPU, allocated by the loader with the
// code object and held until the process ends. In host code `scratch` only names the symbol;
// its device address on the current GPU comes from hipGetSymbolAddress (kept per device).
namespace {
constexpr size_t kNoallocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;  // index: HIP device id; nullptr until looked up

moe_status scratch_on_current_device(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "moe_decode_noalloc: hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "moe_decode_noalloc: hipGetSymbolAddress");
    if (!p) return fail(MOE_E_HIP, "moe_decode_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_decode_noalloc(const moe_layer *layer, const void *x, void *y,
                              const void *residual, void *stream) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (!x || !y || !aligned16(x) || !aligned16(y))
    return fail(MOE_E_INVALID, "x and y must be non-NULL and 16-byte aligned");
  if (residual && !aligned16(residual)) return fail(MOE_E_INVALID, "residual misaligned");
  const Plan p = make_plan(layer, 1);
  if (p.total > kNoallocScratchBytes)
    return fail(MOE_E_WORKSPACE,
                "moe_decode_noalloc: this layer needs %zu bytes of scratch, the library holds %zu "
                "(use moe_decode with a workspace)",
                p.total, kNoallocScratchBytes);
  void *ws = nullptr;
  if ((st = scratch_on_current_device(&ws))) return st;
  return decode_impl(layer, x, y, residual, ws, p, static_cast<hipStream_t>(stream));
}

moe_status moe_stack_workspace_bytes(const moe_layer *layers, int32_t n_layers,
                                     int64_t chunk_tokens, size_t *bytes) {
  g_err.clear();
  if (!bytes) return fail(MOE_E_INVALID, "bytes is NULL");
  StackPlan sp;
  const moe_status st = stack_plan(layers, n_layers, chunk_tokens, &sp);
  if (st) return st;
  *bytes = sp.total;
  return MOE_OK;
}

moe_status moe_stack_forward(const moe_layer *layers, int32_t n_layers, void *h, int64_t T,
                             int64_t chunk_tokens, float eps, void *ws, size_t ws_bytes,
                             void *stream) {
  g_err.clear();
  StackPlan sp;
  moe_status st = stack_plan(layers, n_layers, chunk_tokens, &sp);
  if (st) return st;
  if (T < 0 || T > kMaxTokens) return fail(MOE_E_INVALID, "T %lld out of range", (long long)T);
  if (!(eps >= 0.f)) return fail(MOE_E_INVALID, "eps must be >= 0");
  if (T == 0) return MOE_OK;
  if (!h || !aligned16(h)) return fail(MOE_E_INVALID, "h must be non-NULL and 16-byte aligned");
  if (!ws || !aligned16(ws)) return fail(MOE_E_INVALID, "workspace must be 16-byte aligned");
  if (ws_bytes < sp.total)
    return fail(MOE_E_WORKSPACE, "workspace holds %zu bytes, the stack needs %zu", ws_bytes,
                sp.total);
  for (int32_t l = 0; l < n_layers; ++l)
    if (layers[l].w_format == MOE_W_INT4_G64 && T > 1 && (st = check_tiled(&layers[l])))
      return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = layers[0].hidden;
  const bool bf16 = layers[0].act_dtype == MOE_ACT_BF16;
  const size_t row_bytes = (size_t)H * (bf16 ? 2 : 4);
  void *norm = at<void>(ws, sp.norm);
  void *lws = at<void>(ws, sp.layer_ws);
  // each chunk of rows goes through every layer before the next chunk starts
  for (int64_t r0 = 0; r0 < T; r0 += chunk_tokens) {
    const int64_t n = std::min<int64_t>(chunk_tokens, T - r0);
    void *hc = static_cast<char *>(h) + (size_t)r0 * row_bytes;
    for (int32_t l = 0; l < n_layers; ++l) {
      const Plan p = make_plan(&layers[l], n);
      if (T == 1 && decode_fast(&layers[l])) {
        // the three decode kernels normalise x themselves: no separate RMSNorm launch
        if ((st = decode_impl(&layers[l], hc, hc, hc, lws, p, s, eps))) return st;
        continue;
      }
      hipError_t e = moe::launch_rmsnorm(hc, n, H, eps, bf16, norm, s);
      if (e != hipSuccess) return hip_fail(e, "moe_stack_forward rmsnorm");
      st = (T == 1) ? decode_impl(&layers[l], norm, hc, hc, lws, p, s)
                    : prefill_impl(&layers[l], norm, n, hc, hc, nullptr, lws, p, s);
      if (st) return st;
    }
  }
  return MOE_OK;
}

// ---- decode attention ---------------------------------------------------------------------
namespace {
size_t attn_ws_bytes(int32_t n_q, int64_t max_ctx) {
  int ns;
  int64_t tps;
  moe::attn_plan(max_ctx, 1, &ns, &tps);  // one head group bounds the block count
  return (size_t)ns * n_q * (256 + 2) * 4;
}

moe_status attn_impl(const void *q, const void *k, const void *v, int32_t n_q, int32_t n_kv,
                     int32_t D, int64_t ctx, int64_t stride, float scale, void *out, void *ws,
                     size_t ws_bytes, void *stream, bool packed) {
  g_err.clear();
  if (!moe::attn_supported(n_q, n_kv, D))
    return fail(MOE_E_UNSUPPORTED, "attention needs head_dim 256 and n_q / n_kv in {1,2,4,8}");
  if (ctx < 1 || ctx > (int64_t(1) << 31)) return fail(MOE_E_INVALID, "ctx %lld out of range",
                                                       (long long)ctx);
  if (stride < ctx * D || stride % 8)
    return fail(MOE_E_INVALID, "kv_head_stride must be >= ctx * head_dim and a multiple of 8");
  if (!q || !k || !v || !out || !ws)
    return fail(MOE_E_INVALID, "q, k_cache, v_cache, out and ws must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ws))
    return fail(MOE_E_INVALID, "attention pointers must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(MOE_E_INVALID, "scale must be finite");
  const int G = n_q / n_kv;
  const int hp = packed ? G : 1;
  moe::AttnArgs a{};
  moe::attn_plan(ctx, n_kv, &a.n_split, &a.tps);  // the packed path's blocks, for both
  const size_t need = (size_t)a.n_split * n_q * (D + 2) * 4;
  if (ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "workspace %zu bytes < %zu needed for ctx=%lld", ws_bytes, need,
                (long long)ctx);
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.head_stride = stride;
  a.ctx = ctx;
  a.n_q = n_q;
  a.G = G;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.part_acc = static_cast<float *>(ws);
  a.part_m = a.part_acc + (size_t)a.n_split * n_q * D;
  a.part_l = a.part_m + (size_t)a.n_split * n_q;
  a.out = static_cast<uint16_t *>(out);
  const hipError_t e = moe::launch_attn_decode(a, hp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_attn_decode");
  return MOE_OK;
}
}  // namespace

moe_status moe_attn_workspace_bytes(int32_t n_q, int32_t n_kv, int32_t head_dim, int64_t max_ctx,
                                    size_t *bytes) {
  g_err.clear();
  if (!bytes) return fail(MOE_E_INVALID, "bytes is NULL");
  if (!moe::attn_supported(n_q, n_kv, head_dim))
    return fail(MOE_E_UNSUPPORTED, "attention needs head_dim 256 and n_q / n_kv in {1,2,4,8}");
  if (max_ctx < 1 || max_ctx > (int64_t(1) << 31))
    return fail(MOE_E_INVALID, "max_ctx %lld out of range", (long long)max_ctx);
  *bytes = attn_ws_bytes(n_q, max_ctx);
  return MOE_OK;
}

moe_status moe_attn_decode(const void *q, const void *k_cache, const void *v_cache, int32_t n_q,
                           int32_t n_kv, int32_t head_dim, int64_t ctx, int64_t kv_head_stride,
                           float scale, void *out, void *ws, size_t ws_bytes, void *stream) {
  return attn_impl(q, k_cache, v_cache, n_q, n_kv, head_dim, ctx, kv_head_stride, scale, out, ws,
                   ws_bytes, stream, true);
}

moe_status moe_attn_decode_unpacked(const void *q, const void *k_cache, const void *v_cache,
                                    int32_t n_q, int32_t n_kv, int32_t head_dim, int64_t ctx,
                                    int64_t kv_head_stride, float scale, void *out, void *ws,
                                    size_t ws_bytes, void *stream) {
  return attn_impl(q, k_cache, v_cache, n_q, n_kv, head_dim, ctx, kv_head_stride, scale, out, ws,
                   ws_bytes, stream, false);
}

moe_status moe_gdn_scan(const void *q, const void *k, const void *v, const float *alpha,
                        const float *beta, int64_t T, int32_t n_k, int32_t n_v, int32_t d_k,
                        int32_t d_v, float *state, void *out, void *stream) {
  g_err.clear();
  if (!moe::gdn_supported(n_k, n_v, d_k, d_v))
    return fail(MOE_E_UNSUPPORTED, "DeltaNet scan needs d_k = d_v = 128 and n_v a multiple of n_k");
  if (T < 0 || T > kMaxTokens) return fail(MOE_E_INVALID, "T %lld out of range", (long long)T);
  if (!state) return fail(MOE_E_INVALID, "state must be non-NULL");
  if (T == 0) return MOE_OK;  // the state stays S_0
  if (!q || !k || !v || !alpha || !beta || !out)
    return fail(MOE_E_INVALID, "q, k, v, alpha, beta and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(state) ||
      ((uintptr_t)alpha & 3) || ((uintptr_t)beta & 3))
    return fail(MOE_E_INVALID, "DeltaNet pointers misaligned");
  moe::GdnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.alpha = alpha;
  a.beta = beta;
  a.T = T;
  a.n_k = n_k;
  a.n_v = n_v;
  a.state = state;
  a.out = static_cast<uint16_t *>(out);
  const hipError_t e = moe::launch_gdn_scan(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_gdn_scan");
  return MOE_OK;
}

moe_status moe_gdn_chunked_workspace_bytes(int64_t max_tokens, int32_t n_k, int32_t n_v,
                                           int32_t d_k, int32_t d_v, size_t *bytes) {
  g_err.clear();
  if (!bytes) return fail(MOE_E_INVALID, "bytes is NULL");
  if (!moe::gdn_supported(n_k, n_v, d_k, d_v))
    return fail(MOE_E_UNSUPPORTED, "DeltaNet scan needs d_k = d_v = 128 and n_v a multiple of n_k");
  if (max_tokens < 0 || max_tokens > kMaxTokens)
    return fail(MOE_E_INVALID, "max_tokens %lld out of range", (long long)max_tokens);
  *bytes = moe::gdn_chunk_ws_bytes(max_tokens, n_v);
  return MOE_OK;
}

moe_status moe_gdn_scan_chunked(const void *q, const void *k, const void *v, const float *alpha,
                                const float *beta, int64_t T, int32_t n_k, int32_t n_v,
                                int32_t d_k, int32_t d_v, float *state, void *out, void *ws,
                                size_t ws_bytes, void *stream) {
  g_err.clear();
  if (!moe::gdn_supported(n_k, n_v, d_k, d_v))
    return fail(MOE_E_UNSUPPORTED, "DeltaNet scan needs d_k = d_v = 128 and n_v a multiple of n_k");
  if (T < 0 || T > kMaxTokens) return fail(MOE_E_INVALID, "T %lld out of range", (long long)T);
  if (!state) return fail(MOE_E_INVALID, "state must be non-NULL");
  if (T == 0) return MOE_OK;  // the state stays S_0
  if (!q || !k || !v || !alpha || !beta || !out || !ws)
    return fail(MOE_E_INVALID, "q, k, v, alpha, beta, out and ws must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(state) ||
      !aligned16(ws) || ((uintptr_t)alpha & 3) || ((uintptr_t)beta & 3))
    return fail(MOE_E_INVALID, "DeltaNet pointers misaligned");
  const size_t need = moe::gdn_chunk_ws_bytes(T, n_v);
  if (ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "workspace %zu bytes < %zu needed for T=%lld", ws_bytes, need,
                (long long)T);
  moe::GdnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.alpha = alpha;
  a.beta = beta;
  a.T = T;
  a.n_k = n_k;
  a.n_v = n_v;
  a.state = state;
  a.out = static_cast<uint16_t *>(out);
  a.ws = static_cast<float *>(ws);
  a.nch = (int)((T + 31) / 32);
  const hipError_t e = moe::launch_gdn_chunked(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_gdn_scan_chunked");
  return MOE_OK;
}

moe_status moe_rmsnorm(const void *h, int64_t T, int32_t hidden, float eps, int32_t act_dtype,
                       void *out, void *stream) {
  g_err.clear();
  if (!h || !out) return fail(MOE_E_INVALID, "h and out must be non-NULL");
  if (T < 0 || T > kMaxTokens || hidden <= 0)
    return fail(MOE_E_INVALID, "bad T or hidden");
  if (!(eps >= 0.f)) return fail(MOE_E_INVALID, "eps must be >= 0");
  if (act_dtype != MOE_ACT_BF16 && act_dtype != MOE_ACT_F32)
    return fail(MOE_E_INVALID, "unknown act_dtype %d", act_dtype);
  if (T == 0) return MOE_OK;
  const hipError_t e = moe::launch_rmsnorm(h, T, hidden, eps, act_dtype == MOE_ACT_BF16, out,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_rmsnorm");
  return MOE_OK;
}

moe_status moe_decode_read_ceiling(const moe_layer *layer, const int32_t *ids, int32_t part,
                                   uint32_t *sink, void *stream) {
  g_err.clear();
  moe_status st = check_layer(layer);
  if (st) return st;
  if (!decode_fast(layer))
    return fail(MOE_E_UNSUPPORTED, "read ceilings exist for the packed decode-shaped layer only");
  if (part < 0 || part > 2) return fail(MOE_E_INVALID, "part must be 0, 1 or 2");
  if (!sink || (part > 0 && !ids)) return fail(MOE_E_INVALID, "ids and sink must be non-NULL");
  moe::DecodeArgs da{};
  da.x = static_cast<const uint16_t *>(static_cast<const void *>(layer->router_w));
  da.router_w = layer->router_w;
  da.wt = weights_of(layer);
  da.sel_ids = const_cast<int32_t *>(ids);
  da.H = layer->hidden;
  da.I = layer->inter;
  da.E = layer->n_experts;
  da.k = layer->top_k;
  da.S = layer->n_shared;
  da.T = 1;
  const hipError_t e = moe::launch_read_ceiling(da, part, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_decode_read_ceiling");
  return MOE_OK;
}

moe_status moe_mfma_ceiling(int32_t iters, int32_t operands, uint32_t *sink, double *flops,
                            void *stream) {
  g_err.clear();
  if (iters < 1 || !sink || !flops) return fail(MOE_E_INVALID, "iters >= 1, sink and flops needed");
  if (operands != MOE_CEIL_FULL_MANTISSA && operands != MOE_CEIL_LOW_ENTROPY)
    return fail(MOE_E_INVALID, "unknown operand kind %d", operands);
  *flops = (double)moe::kMfmaCeilingWG * 4 * iters * 8 * 32768.0;
  const hipError_t e = moe::launch_mfma_ceiling(iters, operands == MOE_CEIL_LOW_ENTROPY, sink,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_mfma_ceiling");
  return MOE_OK;
}

moe_status moe_profile_enable(int32_t on) {
  g_err.clear();
  g_prof_on.store(on != 0);
  return MOE_OK;
}

moe_status moe_profile_query(const char *kernel, double *total_ms, int64_t *launches) {
  g_err.clear();
  if (!kernel || !total_ms || !launches) return fail(MOE_E_INVALID, "NULL argument");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double sum = 0.0;
  int64_t n = 0;
  for (ProfRec &r : g_prof) {
    if (r.name != kernel) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "moe_profile_query");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "moe_profile_query");
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return MOE_OK;
}

moe_status moe_profile_reset(void) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (ProfRec &r : g_prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  return MOE_OK;
}

}  // extern "C"
