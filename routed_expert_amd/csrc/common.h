// common.h -- device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kWave = 64;
constexpr int kGroup = 64;        // int4 quantisation group (weights per scale/bias)
constexpr int kRouteBlock = 64;   // tokens per routing block (histogram granularity)
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;
constexpr int kTileM = 128;       // rows of a grouped-GEMM tile (the tallest)
constexpr int kGemmSlots = 512;   // grouped-GEMM workgroups resident at once (256 CUs x 2)
// 32-row blocks per resident gate/up workgroup slot of one N tile (I / 128 N tiles)
inline int gemm_fill(int I) {
  const int n = I >= 256 ? I / 128 : 1;
  return kGemmSlots / n > 0 ? kGemmSlots / n : 1;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
MOE_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round to nearest even; gfx950 lowers this to v_cvt_pk_bf16_f32.
MOE_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Round a double to the nearest bf16, ties to even, in one step (no detour through fp32):
// the mantissa is cut at 7 explicit bits with the usual carry trick on the integer bits,
// which is exact; below 2^-126 the bf16 subnormal grid (spacing 2^-133) applies, past the
// bf16 range the result is +-inf. The rounded value has at most 8 significant bits, so the
// conversion to fp32 that extracts its top half is exact (and gives inf at or past 2^128).
// Both results are formed and one is selected, with no branch: callers round many values
// per thread, and a branch per value costs more than the few extra instructions.
MOE_DEV uint16_t f64_to_bf16_rne(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  // |v| >= 2^-126
  const uint64_t r =
      (mag + 0x00000FFFFFFFFFFFull + ((mag >> 45) & 1ull)) & ~0x00001FFFFFFFFFFFull;
  const uint32_t nb = __float_as_uint((float)__longlong_as_double((long long)r)) >> 16;
  // |v| < 2^-126: the nearest multiple m of 2^-133 (0..128; 128 is the smallest normal),
  // built as bits so that no fp32 subnormal is formed; a value that rounds to zero keeps its
  // sign (the clamp only keeps the conversion defined for the values this branch discards)
  const uint32_t sb = (uint32_t)__builtin_fmin(
      __builtin_rint(__longlong_as_double((long long)mag) * 0x1p133), 256.0);
  const uint32_t m = mag < 0x3810000000000000ull ? sb : nb;
  return mag > 0x7FF0000000000000ull ? (uint16_t)0x7FC0 : (uint16_t)(sign | m);  // NaN
}

// Round to nearest even fp16 (v_cvt_pk_f16_f32). Values outside the fp16 range
// become +-inf; callers keep operands inside it.
MOE_DEV uint32_t pack_f16x2(float lo, float hi) {
  f16x2_t v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
// fp16 pair (w * lo, w * hi), each product rounded once (to nearest even) from its exact
// value: v_fma_mix with f32 sources and a zero addend, the low half then the high half
MOE_DEV uint32_t mul_pack_f16x2(float w, float lo, float hi) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0\n\tv_fma_mixhi_f16 %0, %1, %3, 0"
      : "=&v"(r)
      : "v"(w), "v"(lo), "v"(hi));
  return r;
}

MOE_DEV float f16lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
MOE_DEV float f16hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }

// Two bf16 values (one 32-bit word) to two fp16 values; exact inside the fp16 range.
MOE_DEV uint32_t bf16x2_to_f16x2(uint32_t w) { return pack_f16x2(bf16lo(w), bf16hi(w)); }

// The 8 codes held in one 32-bit word, element order: byte0.lo, byte0.hi, byte1.lo, ...
// q[0..7] receive the codes as floats.
MOE_DEV void unpack8(uint32_t w, float q[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  q[0] = (float)(lo & 0xFF);
  q[1] = (float)(hi & 0xFF);
  q[2] = (float)((lo >> 8) & 0xFF);
  q[3] = (float)((hi >> 8) & 0xFF);
  q[4] = (float)((lo >> 16) & 0xFF);
  q[5] = (float)((hi >> 16) & 0xFF);
  q[6] = (float)(lo >> 24);
  q[7] = (float)(hi >> 24);
}

// K order inside every 8-element chunk of the fp16 operand rows of the grouped GEMMs
// (the copy of x and h): position p holds element kChunkOrder[p] = 0,4,1,5,2,6,3,7. It
// is the order in which dequant8_pk_q produces the eight weights of one 32-bit code word,
// so A and B operands agree without shuffles. kChunkPos is the inverse map.
__device__ constexpr int kChunkPos[8] = {0, 2, 4, 6, 1, 3, 5, 7};

MOE_DEV uint32_t and_or(uint32_t v, uint32_t mask, uint32_t bits) {
  // (v & mask) | bits in one v_and_or_b32 (the compiler emits two instructions here)
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(bits));
  return r;
}

// Eight codes of one 32-bit word to fp16 weights w = fp16_rne(s * q + b), packed math: a
// nibble pair OR-ed into 0x6400 is the fp16 pair (1024 + q_lo, 1024 + q_hi); subtracting
// 1024 is exact, and one fused multiply-add rounds s*q + b once. Output pairs are
// (q0,q4), (q1,q5), (q2,q6), (q3,q7). One shift serves the word: the nibbles at bits 0..3
// and 16..19 (of w and of w >> 8) are taken as they are, those at bits 4..7 and 20..23 are
// masked in place, giving (1024 + 16 q_lo, 1024 + 16 q_hi), and scaled by s / 16 (s2q)
// instead of s. 16 q (s / 16) equals q s exactly when s / 16 is exact in fp16, which holds
// for bf16 scales with |s| >= 2^-13, so every weight gets the same single rounding as with a
// shift per nibble. s2 / s2q / b2 hold their value twice; scale and bias must be
// representable in fp16 (true for bf16 values in [2^-14, 65504]).
MOE_DEV uint4 dequant8_pk_q(uint32_t w, f16x2_t s2, f16x2_t s2q, f16x2_t b2) {
  constexpr uint32_t kLo = 0x000F000Fu, kHi = 0x00F000F0u, kMagic = 0x64006400u;
  const f16x2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const uint32_t u = w >> 8;
  const uint32_t t0 = and_or(w, kLo, kMagic), t1 = and_or(w, kHi, kMagic);
  const uint32_t t2 = and_or(u, kLo, kMagic), t3 = and_or(u, kHi, kMagic);
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
                                         __builtin_bit_cast(f16x2_t, t0) - k1024, s2, b2));
  r.y = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
                                         __builtin_bit_cast(f16x2_t, t1) - k1024, s2q, b2));
  r.z = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
                                         __builtin_bit_cast(f16x2_t, t2) - k1024, s2, b2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
                                         __builtin_bit_cast(f16x2_t, t3) - k1024, s2q, b2));
  return r;
}

// Eight bf16 values (natural order) to eight fp16 values in kChunkOrder.
MOE_DEV uint4 bf16x8_to_f16x8_chunk(uint4 u) {
  uint4 h;
  h.x = pack_f16x2(bf16lo(u.x), bf16lo(u.z));
  h.y = pack_f16x2(bf16hi(u.x), bf16hi(u.z));
  h.z = pack_f16x2(bf16lo(u.y), bf16lo(u.w));
  h.w = pack_f16x2(bf16hi(u.y), bf16hi(u.w));
  return h;
}

// v(l) + v(l ^ M) on every lane l, without the LDS crossbar (__shfl_xor is a ds_bpermute):
//   M = 1, 2: DPP quad permutations (1,0,3,2) and (2,3,0,1);
//   M = 4: DPP rotation by 4 inside each row of 16 lanes; it stands for lane l ^ 4 only
//          when v is already equal on lanes l and l ^ 8, i.e. right after an xor-8 step;
//   M = 8: DPP rotation by 8 inside each row of 16 lanes (lane l reads lane l ^ 8);
//   M = 16, 32: v_permlane16_swap / v_permlane32_swap with v in both operands return the
//          even and the odd rows (the low and the high 32 lanes), each replicated over the
//          pair, so their sum is v(l) + v(l ^ M).
// Addition is commutative, so every lane gets the same bits as v(l) + v(l ^ M).
template <int M>
MOE_DEV uint32_t xor_peer_dpp(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "DPP exchange distance");
  constexpr int ctl = M == 1 ? 0xB1 : M == 2 ? 0x4E : M == 4 ? 0x124 : 0x128;
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctl, 0xF, 0xF, false);
}

template <int M, typename T>
MOE_DEV T xor_sum(T v) {
  static_assert(sizeof(T) == 4, "32-bit values");
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(T, (uint32_t)p[0]) + __builtin_bit_cast(T, (uint32_t)p[1]);
  } else if constexpr (M == 32) {
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(T, (uint32_t)p[0]) + __builtin_bit_cast(T, (uint32_t)p[1]);
  } else {
    return v + __builtin_bit_cast(T, xor_peer_dpp<M>(u));
  }
}

// The same step for a double: both of its 32-bit halves take the same lane permutation.
template <int M>
MOE_DEV double xor_sum_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  auto join = [](uint32_t l, uint32_t h) {
    return __longlong_as_double((long long)(((uint64_t)h << 32) | l));
  };
  if constexpr (M == 16) {
    const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    return join((uint32_t)pl[0], (uint32_t)ph[0]) + join((uint32_t)pl[1], (uint32_t)ph[1]);
  } else if constexpr (M == 32) {
    const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    return join((uint32_t)pl[0], (uint32_t)ph[0]) + join((uint32_t)pl[1], (uint32_t)ph[1]);
  } else {
    return v + join(xor_peer_dpp<M>(lo), xor_peer_dpp<M>(hi));
  }
}

// Sum over the wave, reduction order 32, 16, 8, 4, 2, 1 (xor 4 as a rotation is exact here:
// after the xor-8 step v is equal on lanes l and l ^ 8).
MOE_DEV float wave_sum(float v) {
  v = xor_sum<32>(v);
  v = xor_sum<16>(v);
  v = xor_sum<8>(v);
  v = xor_sum<4>(v);
  v = xor_sum<2>(v);
  return xor_sum<1>(v);
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
MOE_DEV float group_sum(float v) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

MOE_DEV float silu(float v) { return v / (1.0f + expf(-v)); }
// silu from the hardware exp2 and reciprocal (about 1 ulp each), for results that are
// rounded to fp16 anyway: v / (1 + 2^(-v log2 e)).
MOE_DEV float silu_fast(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * 1.4426950408889634f));
}

// ---- wave-wide reductions on the DPP path (no LDS traffic) --------------------------------
// Inclusive-scan pattern: row shifts by 1, 2, 4, 8 inside each row of 16 lanes, then row
// broadcasts of lanes 15 and 31; lane 63 ends with the result, which is broadcast.
template <typename Op>
MOE_DEV uint32_t wave_reduce_u32(uint32_t v, uint32_t identity, Op op) {
  const int id = (int)identity;
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xa, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

MOE_DEV float wave_sum_dpp(float v) {
  const uint32_t r = wave_reduce_u32(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  });
  return __uint_as_float(r);
}

// Sum over a workgroup of 512 threads of each thread's fp64 partial, in one fixed order:
// xor butterfly inside each wave (32, 16, 8, 4, 2, 1; every lane ends with the same bits),
// then the eight wave totals in wave order. red8 holds 8 doubles of LDS. Every thread
// returns the total. The butterfly moves the doubles by DPP and lane swaps instead of the
// LDS crossbar: it is one dependent chain on the stacked decode step's critical path.
MOE_DEV double block512_sum_f64(double v, double *red8) {
  v = xor_sum_f64<32>(v);
  v = xor_sum_f64<16>(v);
  v = xor_sum_f64<8>(v);
  v = xor_sum_f64<4>(v);
  v = xor_sum_f64<2>(v);
  v = xor_sum_f64<1>(v);
  if ((threadIdx.x & 63) == 0) red8[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red8[0];
#pragma unroll
  for (int w = 1; w < 8; ++w) t += red8[w];
  return t;
}

// 1 / sqrt(mean of squares + eps) of a row of H values in fp64. Thread t of the 512 owns
// elements 4t .. 4t+3 of every 2048-element stretch (its partial is the fma chain over them in
// index order), so a kernel that holds those four elements of an H = 2048 row per thread gets
// the same bits as the RMSNorm kernel.
MOE_DEV double row_inv_rms_f64(double partial_ss, int H, double eps, double *red8) {
  const double total = block512_sum_f64(partial_ss, red8);
  return 1.0 / sqrt(total / (double)H + eps);
}

// Order-preserving map of a float to an unsigned key (larger float, larger key).
MOE_DEV uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Order within a wave's LDS scratch: a release/acquire pair at wavefront scope keeps the
// compiler from moving LDS accesses across it; LDS operations of one wave complete in
// order.
MOE_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kTopkScratch = 64 + 4 * kMaxTopK + kMaxTopK;  // uint64 entries per wave

// Top-k of up to 256 logits in one wave: lane l holds experts l, l+64, l+128, l+192 (NaN
// read as -inf, experts >= E excluded). The order is (logit desc, id asc), encoded in one
// 64-bit key: float key in the high word, ~id in the low word. Each lane sorts its four
// keys; the k best elements lie in the k lanes whose heads rank highest, so the wave
// ranks the 64 heads, gathers those lanes' 4k keys and ranks them. Lane j < k then takes
// the j-th largest: it returns its expert id, its position among the k ids in ascending
// id order, and its weight, the softmax over the selected logits (hardware exp2; the
// denominator is summed over the k lanes in a fixed order). Needs E >= k.
// scratch: kTopkScratch uint64 entries of LDS private to the calling wave (16-B aligned).
MOE_DEV void wave_topk(const float v[4], int E, int k, uint64_t *scratch, int &id_out,
                       int &pos_out, float &w_out) {
  const int lane = threadIdx.x & 63;
  uint64_t key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    const float f = v[c] != v[c] ? -INFINITY : v[c];
    // real experts have a nonzero high word (float key of -inf is > 0); 0 = absent
    key[c] = e < E ? ((uint64_t)float_key(f) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e)
                   : 0ull;
  }
#define MOE_CSWAP(a, b)                                          \
  if (key[b] > key[a]) {                                         \
    const uint64_t t_ = key[a];                                  \
    key[a] = key[b];                                             \
    key[b] = t_;                                                 \
  }
  MOE_CSWAP(0, 1) MOE_CSWAP(2, 3) MOE_CSWAP(0, 2) MOE_CSWAP(1, 3) MOE_CSWAP(1, 2)
#undef MOE_CSWAP
  uint64_t *heads = scratch, *cand = scratch + 64, *best = scratch + 64 + 4 * kMaxTopK;
  heads[lane] = key[0];
  if (lane < 4 * kMaxTopK) cand[lane] = 0ull;  // unused candidate slots rank last
  wave_lds_sync();
  int r = 0;
#pragma unroll 8
  for (int q = 0; q < 64; q += 2) {
    const ulonglong2 h2 = *reinterpret_cast<const ulonglong2 *>(heads + q);
    r += (h2.x > key[0]) + (h2.y > key[0]);
  }
  if (r < k) {
#pragma unroll
    for (int c = 0; c < 4; ++c) cand[4 * r + c] = key[c];
  }
  wave_lds_sync();
  {
    const uint64_t mine = cand[lane & (4 * kMaxTopK - 1)];
    int r2 = 0;
#pragma unroll
    for (int q = 0; q < 4 * kMaxTopK; q += 2) {
      const ulonglong2 c2 = *reinterpret_cast<const ulonglong2 *>(cand + q);
      r2 += (c2.x > mine) + (c2.y > mine);
    }
    if (lane < 4 * kMaxTopK && mine != 0ull && r2 < k) best[r2] = mine;
  }
  wave_lds_sync();
  // lane j < k: the j-th largest key; every such lane reads all k winners (same order)
  uint64_t win[kMaxTopK];
#pragma unroll
  for (int q = 0; q < kMaxTopK; q += 2) {
    const ulonglong2 b2 = *reinterpret_cast<const ulonglong2 *>(best + q);
    win[q] = b2.x;
    win[q + 1] = b2.y;
  }
  wave_lds_sync();  // scratch may be reused by the caller's next token
  uint64_t mw = win[0];
#pragma unroll
  for (int q = 1; q < kMaxTopK; ++q)
    if (q == lane) mw = win[q];
  const int id = (int)(0xFFFFFFFFu - (uint32_t)mw);
  const float top = key_float((uint32_t)(win[0] >> 32));
  float den = 0.f, mine = 0.f;
  int pos = 0;
#pragma unroll
  for (int q = 0; q < kMaxTopK; ++q) {
    if (q < k) {
      const float vq = key_float((uint32_t)(win[q] >> 32));
      // exp(v - top) from the hardware exp2; top == -inf only when every logit is -inf
      const float ex = top == -INFINITY ? 1.0f
                                        : __builtin_amdgcn_exp2f((vq - top) * 1.4426950408889634f);
      den += ex;
      if (q == lane) mine = ex;
      pos += (int)(0xFFFFFFFFu - (uint32_t)win[q]) < id ? 1 : 0;
    }
  }
  id_out = id;
  pos_out = pos;
  w_out = mine / den;
}

}  // namespace moe
