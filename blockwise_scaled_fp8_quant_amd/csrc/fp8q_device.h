// Device helpers shared by the gfx950 kernels of the blockwise FP8 layer.
//
// Element rule (page "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung mit
// End-to-End FP8-Praezisionstraining", section "Der technische Durchbruch": E4M3
// codes with one scale per block; +-448 from page "FP8 Trainingsinfrastructuur",
// section "Het landschap van numerieke precisie"):
//     q = E4M3_RNE_SAT(RN_fp32(x / s))
// with s = RN_fp32(amax / 448) (amax mode) or the smallest power of two with
// 448 * s >= amax (pow2 mode, page 1, section "Warum dies fuer die
// KI-Oekonomie wichtig ist"), s = 1 for an all-zero block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

enum { kModeAmax = 0, kModePow2 = 1 };

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read once: non-temporal hint).
__device__ __forceinline__ uint4 load_stream16(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Streaming stores, for codes that are written once and read only much later
// (quantized weights): the non-temporal hint lets the write stream pass the
// caches (measured on gfx950: ~6% more HBM bandwidth for the weight quantizer
// than plain stores).  Activation codes, read by the very next GEMM, use
// plain stores and may stay in the caches.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_stream8(void *p, uint2 v) {
  const u32x2_t x = {v.x, v.y};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x2_t *>(p));
}
__device__ __forceinline__ void store_stream16(void *p, uint4 v) {
  const u32x4_t x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t *>(p));
}

// bf16 halves of a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// max(|a|, |b|, c) -- one v_max3_f32 with abs source modifiers.
__device__ __forceinline__ float max3_abs(float c, float a, float b) {
  return __builtin_fmaxf(c, __builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(b)));
}

// Running |max| over the 8 bf16 values of a 16-byte chunk.
__device__ __forceinline__ float chunk_absmax(const uint4 &v, float m) {
  m = max3_abs(m, bf16_lo(v.x), bf16_hi(v.x));
  m = max3_abs(m, bf16_lo(v.y), bf16_hi(v.y));
  m = max3_abs(m, bf16_lo(v.z), bf16_hi(v.z));
  m = max3_abs(m, bf16_lo(v.w), bf16_hi(v.w));
  return m;
}

// Cross-lane max through DPP (values are >= 0, so the bit pattern of the
// neighbour is combined with an ordinary fp32 max).
template <int kCtrl>
__device__ __forceinline__ float dpp_max(float v) {
  int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false);
  return __builtin_fmaxf(v, __int_as_float(o));
}
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7-i in each group of 8
constexpr int kDppMirror = 0x140;      // row_mirror: lane i <-> 15-i in each row of 16

// Max over each aligned group of 8 lanes.
__device__ __forceinline__ float group8_max(float v) {
  v = dpp_max<kDppQuadSwap1>(v);
  v = dpp_max<kDppQuadSwap2>(v);
  v = dpp_max<kDppHalfMirror>(v);
  return v;
}

// Max over each aligned row of 16 lanes.
__device__ __forceinline__ float group16_max(float v) {
  v = group8_max(v);
  v = dpp_max<kDppMirror>(v);
  return v;
}

// Per-block quantisation parameters.
//
// amax mode, fast path: y = RN(1/s) once per block, then per element
//     q0 = RN(x*y);  nr = RN(q0*s - x) (fused, exact);  r = RN(q0 - nr*y) (fused)
// -- a remainder correction of the reciprocal-multiply quotient (Markstein,
// "Computation of elementary functions on the IBM RISC System/6000 processor",
// IBM J. Res. Dev. 1990; Muller et al., Handbook of Floating-Point Arithmetic,
// FMA-based division).  The remainder is negated so that x = -0 gives -0.  An
// exhaustive comparison over every pair of bf16 values (x, amax) with
// |x| <= amax shows that the E4M3 byte it yields equals the one from the
// correctly rounded quotient whenever amax >= 2^-104; below that the remainder
// underflows, so blocks with amax < 2^-100 use the IEEE division x / s.
// pow2 mode: x / 2^e is exact (v_ldexp_f32, correctly rounded when the result
// is subnormal).
struct BlockQ {
  float s;   // stored scale
  float y;   // RN(1/s)            (amax mode)
  int e;     // s = 2^e            (pow2 mode)
  bool slow; // use the IEEE division (amax mode, amax < 2^-100)
};

__device__ __forceinline__ int pow2_exponent(float amax) {
  // amax > 0, finite.  amax = m * 2^E with m in [1,2); 448 = 1.75 * 2^8, so the
  // smallest e with 448 * 2^e >= amax is E-8 when m <= 1.75, else E-7.  It is
  // kept at -127 or above, the E8M0 range of a power-of-two scale (448 * 2^-127
  // still covers any smaller amax).
  float a = amax;
  int adj = 0;
  if (a < 0x1p-126f) {  // subnormal: scale up exactly first
    a = a * 0x1p64f;
    adj = 64;
  }
  uint32_t b = __float_as_uint(a);
  int E = (int)(b >> 23) - 127 - adj;
  const int e = ((b & 0x7FFFFFu) <= 0x600000u) ? E - 8 : E - 7;
  return e < -127 ? -127 : e;
}

template <int kMode>
__device__ __forceinline__ BlockQ block_params(float amax) {
  BlockQ p;
  if (kMode == kModeAmax) {
    p.s = (amax == 0.0f) ? 1.0f : amax / 448.0f;  // IEEE division
    p.y = 1.0f / p.s;                             // IEEE division
    p.e = 0;
    p.slow = amax < 0x1p-100f;
  } else {
    p.e = (amax == 0.0f) ? 0 : pow2_exponent(amax);
    p.s = __builtin_ldexpf(1.0f, p.e);  // exact: e in [-127, 120]
    p.y = 0.0f;
    p.slow = false;
  }
  return p;
}

// RN_fp32(x / s) on the fast path.
template <int kMode>
__device__ __forceinline__ float quotient(const BlockQ &p, float x) {
  if (kMode == kModeAmax) {
    float q0 = x * p.y;
    float nr = __builtin_fmaf(q0, p.s, -x);
    return __builtin_fmaf(nr, -p.y, q0);
  } else {
    return __builtin_ldexpf(x, -p.e);
  }
}

// Four fp32 values (already RN(x/s)) -> four E4M3 bytes, little-endian in a
// 32-bit word: clamp to +-448, then the hardware conversion (round to nearest
// even).  The clamp makes saturation explicit; med3 keeps the sign of zero.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Eight bf16 (one 16-byte chunk) -> eight E4M3 bytes.
template <int kMode>
__device__ __forceinline__ uint2 quant_chunk(const BlockQ &p, const uint4 &v) {
  float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float r[8];
  if (kMode == kModeAmax && p.slow) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = f[i] / p.s;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = quotient<kMode>(p, f[i]);
  }
  uint2 o;
  o.x = pack4_e4m3(r[0], r[1], r[2], r[3]);
  o.y = pack4_e4m3(r[4], r[5], r[6], r[7]);
  return o;
}

}  // namespace fp8q
