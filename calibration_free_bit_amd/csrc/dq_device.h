// dq_device.h -- device-side number formats for the DualQuant kernels (gfx950).
//
// Element grids ("DualQuant" paper summary §3: integer formats round and
// clip, floating-point formats take the nearest level of their grid):
//   INT4  integers [-8, 7], round half to even, clip;
//   E2M1  magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, nearest, ties to the even
//         encoding, saturating at 6.
// Scale sets (summary §3; reproduction README "Core equations": the
// projection acts on inverse scales, since not every positive real can be
// stored in the scale format):
//   fp16  IEEE binary16, positive finite;
//   E8M0  2^e, e in [-127, 127];
//   E4M3  OCP E4M3FN without sign: k 2^-9 (k = 1..7) and 2^e (1 + m/8)
//         up to 448.
// Projection takes a positive float64 to the nearest legal value (ties to
// even for fp16 / E4M3, upward for E8M0), clamped to the smallest legal
// value and saturated at the largest.
//
// Requantization x = W / (a b) must be decided on the exact quotient. The
// fast path evaluates y ~= x in float32 from precomputed reciprocals; its
// relative error is at most 7 units of 2^-24, so for |x| <= 8.25 the error
// is below 3.5e-6. Any element whose y lies within 2^-17 of a rounding
// midpoint is flagged, and the caller then re-decides the whole group with
// the exact path: the sign of W - m a b for the candidate midpoint m comes
// from one fused multiply-add, exact because m*a is exact in float32 and
// the FMA rounds W - (m a) b once.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace dq {

enum : int { kGridInt4 = 0, kGridE2M1 = 1, kGridInt8 = 2, kGridE4M3 = 3 };
enum : int { kScaleFp16 = 0, kScaleE8M0 = 1, kScaleE4M3 = 2 };
enum : int { kWF32 = 0, kWBF16 = 1 };

// |y - rint(y)| above this flags a possible misrounding (0.5 - 2^-17), for
// quotients up to 8.25; the int8 grid (quotients up to 127.25) uses
// 0.5 - 2^-13. The estimate's relative error is below 7 * 2^-24.
constexpr float kTieFlag = 0.5f - 0x1p-17f;

// 1 / a, exactly, for a power of two a (float32, subnormals included).
__device__ __forceinline__ float recip_pow2(float a) {
  return __builtin_ldexpf(1.0f, 1 - __builtin_amdgcn_frexp_expf(a));
}
constexpr float kTieFlag8 = 0.5f - 0x1p-13f;

// ------------------------------------------------------------ scale codes

// binade exponent k with 2^k <= x < 2^(k+1), for normal x > 0
__device__ __forceinline__ int binade(double x) { return __builtin_amdgcn_frexp_exp(x) - 1; }

template <int AFMT> struct ScaleStore;
template <> struct ScaleStore<kScaleFp16> { using T = uint16_t; };
template <> struct ScaleStore<kScaleE8M0> { using T = uint8_t; };
template <> struct ScaleStore<kScaleE4M3> { using T = uint8_t; };

// 1 / a for a block scale of format AFMT. E8M0 scales reach 2^-127, a
// float32 subnormal, which the hardware reciprocal does not take, so they
// use the exact power-of-two reciprocal; fp16 (>= 2^-24) and E4M3 (>= 2^-9)
// scales are normal float32 values and take the 1-ulp hardware reciprocal.
template <int AFMT>
__device__ __forceinline__ float recip_scale(float a) {
  if constexpr (AFMT == kScaleE8M0) {
    return recip_pow2(a);
  } else {
    return __builtin_amdgcn_rcpf(a);
  }
}

__device__ __forceinline__ float fp16_bits_to_float(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

template <int AFMT>
__device__ __forceinline__ float decode_scale(typename ScaleStore<AFMT>::T c) {
  if constexpr (AFMT == kScaleFp16) {
    return fp16_bits_to_float(c);
  } else if constexpr (AFMT == kScaleE8M0) {
    return __builtin_ldexpf(1.0f, (int)c - 127);
  } else {
    const int e = c >> 3, m = c & 7;
    return e == 0 ? (float)m * 0x1p-9f : __builtin_ldexpf(1.0f + 0.125f * (float)m, e - 7);
  }
}

// Code of a legal value (the value must already be legal).
template <int AFMT>
__device__ __forceinline__ typename ScaleStore<AFMT>::T encode_scale(double v) {
  if constexpr (AFMT == kScaleFp16) {
    return __half_as_ushort(__float2half_rn((float)v));
  } else if constexpr (AFMT == kScaleE8M0) {
    return (uint8_t)(binade(v) + 127);
  } else {
    if (v < 0x1p-6) return (uint8_t)(v * 512.0);
    const int e = binade(v);
    const int m = (int)((__builtin_ldexp(v, -e) - 1.0) * 8.0);
    return (uint8_t)(((e + 7) << 3) | m);
  }
}

// ------------------------------------------------------------- projection

// Round x > 0 to a multiple of 2^lsb_exp, to nearest even, by adding and
// removing 1.5 * 2^(lsb_exp + 52): the sum's unit in the last place is
// exactly 2^lsb_exp. Needs x < 2^(lsb_exp + 52).
__device__ __forceinline__ double round_to_exp(double x, int lsb_exp) {
  const double c = __builtin_ldexp(1.5, lsb_exp + 52);
  return (x + c) - c;
}


template <int AFMT>
__device__ __forceinline__ double project(double x) {
  if constexpr (AFMT == kScaleFp16) {
    x = __builtin_fmin(__builtin_fmax(x, 0x1p-24), 65504.0);
    const int k = max(binade(x), -14);            // below 2^-14: fixed 2^-24 step
    return round_to_exp(x, k - 10);
  } else if constexpr (AFMT == kScaleE4M3) {
    x = __builtin_fmin(__builtin_fmax(x, 0x1p-9), 448.0);
    const int k = max(binade(x), -6);             // below 2^-6: fixed 2^-9 step
    return round_to_exp(x, k - 3);
  } else {
    x = __builtin_fmax(x, 0x1p-127);
    int k = binade(x);                            // 2^k <= x < 2^(k+1)
    if (x >= __builtin_ldexp(1.5, k)) k += 1;     // nearest; the midpoint goes up
    return __builtin_ldexp(1.0, min(k, 127));
  }
}

// Closed-form least-squares scale with the scale-1 rule for an all-zero
// code slice (den == 0).
template <int AFMT>
__device__ __forceinline__ double ls_scale(double num, double den) {
  return den > 0.0 ? project<AFMT>(num / den) : 1.0;
}

// Certified projection of a float32 estimate of a positive quotient.
// nf / df must be within relative error eps / 1.25 of the exact quotient,
// counting the 1-ulp reciprocal and the product formed here (2^-24 each,
// relative). Operands below 2^-100 are refused, so subnormal roundings
// inside the estimate stay far below that bound. For fp16 and E4M3 the
// hardware conversions (round to nearest even, subnormals kept) project
// both ends of [x (1 - eps), x (1 + eps)], which contains the exact
// (clamped) quotient; rounding is monotone, so equal results at both ends
// are the projection of the exact quotient. For E8M0 the quotient is
// compared with the nearest binade midpoint. Otherwise `unsure` is set and
// the caller must use ls_scale.
template <int AFMT>
__device__ __forceinline__ float project_certified(float nf, float df, float eps, bool& unsure) {
  const float qf = nf * __builtin_amdgcn_rcpf(df);
  // far outside every format's range, or tiny operands: exact path
  if (!(qf > 0x1p-100f && qf < 0x1p100f) || !(df > 0x1p-100f) || !(nf > 0x1p-100f)) {
    unsure = true;
    return 1.0f;
  }
  if constexpr (AFMT == kScaleE8M0) {
    const float x = __builtin_fmaxf(qf, 0x1p-127f);
    const int k = __builtin_amdgcn_frexp_expf(x) - 1;           // 2^k <= x < 2^(k+1)
    const float mid = __builtin_ldexpf(1.5f, k);
    unsure |= __builtin_fabsf(x - mid) <= eps * x;
    return __builtin_ldexpf(1.0f, min(x >= mid ? k + 1 : k, 127));
  } else if constexpr (AFMT == kScaleFp16) {
    const float x = __builtin_amdgcn_fmed3f(qf, 0x1p-24f, 65504.0f);
    const _Float16 rl = (_Float16)(x * (1.0f - eps));
    const _Float16 rh = (_Float16)(x * (1.0f + eps));
    unsure |= __builtin_bit_cast(uint16_t, rl) != __builtin_bit_cast(uint16_t, rh);
    return (float)rl;
  } else {
    // OCP E4M3FN conversion of both ends into bytes 0 and 1 (the upper end
    // stays below 464, where the conversion would give NaN)
    const float x = __builtin_amdgcn_fmed3f(qf, 0x1p-9f, 448.0f);
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(x * (1.0f - eps), x * (1.0f + eps), 0, false);
    unsure |= ((w ^ (w >> 8)) & 0xFF) != 0;
    return __builtin_amdgcn_cvt_f32_fp8(w, 0);
  }
}

// Fast path of ls_scale from float64 sums: the quotient of their float32
// roundings with a 1-ulp reciprocal is within 5 * 2^-24 (relative) of the
// exact quotient, inside the bracket of 2^-20.
constexpr float kScaleSure = 0x1p-20f;

template <int AFMT>
__device__ __forceinline__ float ls_scale_fast(double num, double den, bool& unsure) {
  if (!(den > 0.0)) return 1.0f;
  return project_certified<AFMT>((float)num, (float)den, kScaleSure, unsure);
}

// ------------------------------------------------------- element quantizer

template <int GRID> struct Grid;

// Number of non-zero nibbles / bytes of x.
__device__ __forceinline__ int nibbles_differ(uint32_t x) {
  return __builtin_popcount((x | (x >> 1) | (x >> 2) | (x >> 3)) & 0x11111111u);
}
__device__ __forceinline__ int bytes_differ(uint32_t x) {
  x |= x >> 4;
  return __builtin_popcount((x | (x >> 1) | (x >> 2) | (x >> 3)) & 0x01010101u);
}

template <> struct Grid<kGridInt4> {
  static constexpr float qmax = 7.0f;
  static constexpr int kBits = 4;
  // Fast path: y ~= x. Returns the code; accumulates |y - code| (in units
  // of the grid step) into flag.
  __device__ static __forceinline__ float fast(float y, float& flag) {
    const float yc = __builtin_amdgcn_fmed3f(y, -8.25f, 7.25f);
    const float q = __builtin_rintf(yc);
    flag = __builtin_fmaxf(flag, __builtin_fabsf(yc - q));
    return q;
  }
  // Exact path: y ~= x within 0.5, w = W, ab = a and b with m*a exact.
  __device__ static __forceinline__ float exact(float y, float w, float a, float b) {
    const float yc = __builtin_amdgcn_fmed3f(y, -8.25f, 7.25f);
    const float k = __builtin_floorf(yc);
    const float m = k + 0.5f;
    const float d = __builtin_fmaf(-(m * a), b, w);   // sign of W - m a b, exact
    const bool k_odd = ((int)k & 1) != 0;
    const float up = (d > 0.0f || (d == 0.0f && k_odd)) ? 1.0f : 0.0f;
    return __builtin_amdgcn_fmed3f(k + up, -8.0f, 7.0f);
  }
  // Codes of N estimates; true if any of them may round differently at the
  // exact quotient (then the caller re-decides those with exact(); near()
  // tells which). diff is unused here.
  static constexpr bool kTwoEnded = false;  // one rounding and its residual
  static constexpr bool kSlotMask = false;
  static constexpr bool kScaledEnds = false;
  template <int N>
  __device__ static __forceinline__ bool fast_n(const float* y, float* q, uint32_t* diff, uint32_t* hiw) {
    float flag = 0.0f;
#pragma unroll
    for (int e = 0; e < N; ++e) q[e] = fast(y[e], flag);
    return flag > kTieFlag;
  }
  __device__ static __forceinline__ bool near(const float* y, const float* q, const uint32_t* diff,
                                              int e) {
    return __builtin_fabsf(__builtin_amdgcn_fmed3f(y[e], -8.25f, 7.25f) - q[e]) > kTieFlag;
  }
  // Codes of N quotients that are exact (rounding them is the decision).
  template <int N>
  __device__ static __forceinline__ void nearest_n(const float* y, float* q) {
#pragma unroll
    for (int e = 0; e < N; ++e) q[e] = __builtin_rintf(__builtin_amdgcn_fmed3f(y[e], -8.25f, 7.25f));
  }
  // Nibbles of 8 codes, element k in bits 4k..4k+3 (two's complement). A
  // pair of codes offset by 8 is the byte 16 (q1 + 8) + (q0 + 8), an exact
  // integer in [0, 255] that the byte conversion packs in place; flipping
  // bit 3 of each offset nibble gives the two's complement nibble.
  __device__ static __forceinline__ uint32_t pack8(const float* q) {
    uint32_t w = 0u;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(q[2 * p + 1], 16.0f, q[2 * p] + 136.0f), p, w);
    return w ^ 0x88888888u;
  }
  // 8 codes in storage form, and the number of codes two such words differ in.
  using Word = uint32_t;
  __device__ static __forceinline__ Word encode8(const float* q) { return pack8(q); }
  __device__ static __forceinline__ int count_diff(Word x, Word y) { return nibbles_differ(x ^ y); }
  // Store 8 codes (4 bytes, 4-byte aligned).
  __device__ static __forceinline__ void store8(uint8_t* dst, const float* q) {
    *reinterpret_cast<Word*>(dst) = encode8(q);
  }
};

template <> struct Grid<kGridE2M1> {
  static constexpr float qmax = 6.0f;
  static constexpr int kBits = 4;
  // Exact path. In binade scale t = |y| * 2^s (s = 1 below 2, 0 below 4, -1
  // above) the E2M1 levels are consecutive integers and ties to the even
  // encoding are ties to even on t. frexp_exp gives e with |y| in
  // [2^(e-1), 2^e).
  __device__ static __forceinline__ float exact(float y, float w, float a, float b) {
    const float ay = __builtin_fminf(__builtin_fabsf(y), 6.25f);
    const int s = max(-1, min(1, 2 - __builtin_amdgcn_frexp_expf(ay)));
    const float t = __builtin_ldexpf(ay, s);
    const float k = __builtin_floorf(t);
    const float m = __builtin_ldexpf(k + 0.5f, -s);   // midpoint in |x| units
    const float d = __builtin_fmaf(-(m * a), b, __builtin_fabsf(w));
    const bool k_odd = ((int)k & 1) != 0;
    const float up = (d > 0.0f || (d == 0.0f && k_odd)) ? 1.0f : 0.0f;
    const float mag = __builtin_fminf(__builtin_ldexpf(k + up, -s), 6.0f);
    return __builtin_copysignf(mag, w);
  }
  // gfx950's scaled FP4 conversion rounds a float32 to the nearest E2M1
  // level with ties to the even encoding and saturates at 6 -- the same
  // rule as exact() -- but keeps the sign of a zero result (code 8).
  // Element 2p goes to nibble 2p of the word, 2p + 1 to nibble 2p + 1.
  __device__ static __forceinline__ uint32_t cvt8(const float* y) {
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
    return w;
  }
  // Codes of N estimates (|y - x| below 2^-21 |x|): every value in
  // [y (1 - 2^-20), y (1 + 2^-20)] contains x, and rounding is monotone, so
  // when both ends give the same codes those are the codes of x. Otherwise
  // returns true and the caller re-decides with exact(). A zero code may
  // come back as -0, which is arithmetically harmless.
  // diff[g] receives the differing nibbles of group g (near() reads them),
  // hiw[g] the codes at the upper ends (resolve() reads them).
  template <int N>
  __device__ static __forceinline__ bool fast_n(const float* y, float* q, uint32_t* diff, uint32_t* hiw) {
    static_assert(N % 8 == 0, "groups of 8");
    uint32_t any = 0u;
#pragma unroll
    for (int g = 0; g < N; g += 8) {
      float lo[8], hi[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float yc = __builtin_amdgcn_fmed3f(y[g + k], -8.0f, 8.0f);
        lo[k] = yc * (1.0f - 0x1p-20f);
        hi[k] = yc * (1.0f + 0x1p-20f);
      }
      const uint32_t wl = cvt8(lo), wh = cvt8(hi);
      diff[g / 8] = wl ^ wh;
      hiw[g / 8] = wh;
      any |= wl ^ wh;
      typedef float f2 __attribute__((ext_vector_type(2)));
      f2 r;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wl, 1.0f, 0); q[g + 0] = r.x; q[g + 1] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wl, 1.0f, 1); q[g + 2] = r.x; q[g + 3] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wl, 1.0f, 2); q[g + 4] = r.x; q[g + 5] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wl, 1.0f, 3); q[g + 6] = r.x; q[g + 7] = r.y;
    }
    return any != 0u;
  }
  __device__ static __forceinline__ bool near(const float* y, const float* q, const uint32_t* diff,
                                              int e) {
    return ((diff[e >> 3] >> (4 * (e & 7))) & 0xFu) != 0u;
  }
  // fast_n of the quotients wrb[e] * ra[e / BL] (wrb = W / b, ra = 1 / a,
  // both from 1-ulp reciprocals) without forming them: the two ends come
  // from the block's reciprocal scaled by 1 -+ 2^-20, each within 7 units
  // of 2^-24 of x (1 -+ 2^-20) (two reciprocals, three roundings), so x
  // lies between them. No clamp: the conversion saturates at +-6 for every
  // larger magnitude, infinities included.
  static constexpr bool kScaledEnds = true;
  template <int N, int BL>
  __device__ static __forceinline__ bool fast_scaled(const float* wrb, const float* ra, float* q, uint32_t* diff,
                                                     uint32_t* hiw) {
    static_assert(N % 8 == 0 && (BL % 8 == 0 || 8 % BL == 0), "groups of 8");
    uint32_t any = 0u;
#pragma unroll
    for (int g = 0; g < N; g += 8) {
      float lo[8], hi[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float r = ra[(g + k) / BL];
        lo[k] = wrb[g + k] * (r * (1.0f - 0x1p-20f));
        hi[k] = wrb[g + k] * (r * (1.0f + 0x1p-20f));
      }
      const uint32_t wl = cvt8(lo), wh = cvt8(hi);
      diff[g / 8] = wl ^ wh;
      hiw[g / 8] = wh;
      any |= wl ^ wh;
      typedef float f2 __attribute__((ext_vector_type(2)));
      f2 r;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wl, 1.0f, 0); q[g + 0] = r.x; q[g + 1] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wl, 1.0f, 1); q[g + 2] = r.x; q[g + 3] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wl, 1.0f, 2); q[g + 4] = r.x; q[g + 5] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wl, 1.0f, 3); q[g + 6] = r.x; q[g + 7] = r.y;
    }
    return any != 0u;
  }
  // Rounded by two conversions. Exact ties are the common case of differing
  // ends here and stay rare enough per wave (an element in a few thousand
  // on the workloads) that the re-decision visits only the slots some lane
  // flags, found from the lanes' difference words (kSlotMask): field
  // e % kPerWord of word e / kPerWord.
  static constexpr bool kTwoEnded = true;
  static constexpr bool kSlotMask = true;
  static constexpr int kPerWord = 8;
  __device__ static __forceinline__ uint32_t field(const uint32_t* d, int e) {
    return (d[e >> 3] >> (4 * (e & 7))) & 0xFu;
  }
  // Exact code of element e from the codes at its bracket's ends: ql (the
  // lower magnitude, decoded) and the upper one in hiw. Where they differ
  // the exact quotient |x| is on one side of their midpoint m, or on it:
  // the sign of |W| - m a b decides (m a b is exact: m has at most 3
  // significant bits), a tie goes to the even encoding (the nibble's low
  // bit is the mantissa bit). Where they agree the result is ql.
  __device__ static __forceinline__ float resolve(float ql, const uint32_t* hiw, int e, float w, float a,
                                                  float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const uint32_t wh = hiw[e >> 3];
    f2 r;
    switch ((e & 7) >> 1) {  // e is a compile-time constant at every call
      case 0: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wh, 1.0f, 0); break;
      case 1: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wh, 1.0f, 1); break;
      case 2: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wh, 1.0f, 2); break;
      default: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wh, 1.0f, 3); break;
    }
    const float qh = (e & 1) ? r.y : r.x;
    const float m = 0.5f * (__builtin_fabsf(ql) + __builtin_fabsf(qh));
    const float d = __builtin_fmaf(-(m * a), b, __builtin_fabsf(w));
    const bool hi_even = ((wh >> (4 * (e & 7))) & 1u) == 0u;
    return (d > 0.0f || (d == 0.0f && hi_even)) ? qh : ql;
  }
  // Codes of N quotients that are exact: the conversion's own rounding is
  // the decision (a zero may come back as -0).
  template <int N>
  __device__ static __forceinline__ void nearest_n(const float* y, float* q) {
    static_assert(N % 8 == 0, "groups of 8");
#pragma unroll
    for (int g = 0; g < N; g += 8) {
      float yc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) yc[k] = __builtin_amdgcn_fmed3f(y[g + k], -8.0f, 8.0f);
      const uint32_t w = cvt8(yc);
      typedef float f2 __attribute__((ext_vector_type(2)));
      f2 r;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); q[g + 0] = r.x; q[g + 1] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); q[g + 2] = r.x; q[g + 3] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); q[g + 4] = r.x; q[g + 5] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); q[g + 6] = r.x; q[g + 7] = r.y;
    }
  }
  // Nibbles of 8 codes (exact E2M1 values, so the conversion is exact);
  // a zero is stored as +0.
  __device__ static __forceinline__ uint32_t pack8(const float* q) {
    const uint32_t w = cvt8(q);
    const uint32_t mag = w & 0x77777777u;
    const uint32_t nonzero = (mag + 0x77777777u) & 0x88888888u;  // bit 3 set iff magnitude != 0
    return w & (0x77777777u | nonzero);
  }
  using Word = uint32_t;
  __device__ static __forceinline__ Word encode8(const float* q) { return pack8(q); }
  __device__ static __forceinline__ int count_diff(Word x, Word y) { return nibbles_differ(x ^ y); }
  __device__ static __forceinline__ void store8(uint8_t* dst, const float* q) {
    *reinterpret_cast<Word*>(dst) = encode8(q);
  }
};

template <> struct Grid<kGridInt8> {
  static constexpr float qmax = 127.0f;
  static constexpr int kBits = 8;
  __device__ static __forceinline__ float fast(float y, float& flag) {
    const float yc = __builtin_amdgcn_fmed3f(y, -127.25f, 127.25f);
    const float q = __builtin_rintf(yc);
    flag = __builtin_fmaxf(flag, __builtin_fabsf(yc - q));
    return q;
  }
  // Exact path: y ~= x within 0.5; m*a is exact (m has at most 8 bits).
  __device__ static __forceinline__ float exact(float y, float w, float a, float b) {
    const float yc = __builtin_amdgcn_fmed3f(y, -127.25f, 127.25f);
    const float k = __builtin_floorf(yc);
    const float m = k + 0.5f;
    const float d = __builtin_fmaf(-(m * a), b, w);   // sign of W - m a b, exact
    const bool k_odd = ((int)k & 1) != 0;
    const float up = (d > 0.0f || (d == 0.0f && k_odd)) ? 1.0f : 0.0f;
    return __builtin_amdgcn_fmed3f(k + up, -127.0f, 127.0f);
  }
  static constexpr bool kTwoEnded = false;
  static constexpr bool kSlotMask = false;
  static constexpr bool kScaledEnds = false;
  template <int N>
  __device__ static __forceinline__ bool fast_n(const float* y, float* q, uint32_t* diff, uint32_t* hiw) {
    float flag = 0.0f;
#pragma unroll
    for (int e = 0; e < N; ++e) q[e] = fast(y[e], flag);
    return flag > kTieFlag8;
  }
  __device__ static __forceinline__ bool near(const float* y, const float* q, const uint32_t* diff,
                                              int e) {
    return __builtin_fabsf(__builtin_amdgcn_fmed3f(y[e], -127.25f, 127.25f) - q[e]) > kTieFlag8;
  }
  // Codes of N quotients that are exact (rounding them is the decision).
  template <int N>
  __device__ static __forceinline__ void nearest_n(const float* y, float* q) {
#pragma unroll
    for (int e = 0; e < N; ++e) q[e] = __builtin_rintf(__builtin_amdgcn_fmed3f(y[e], -127.25f, 127.25f));
  }
  // 8 codes as two's complement bytes (8 bytes, 8-byte aligned when stored).
  using Word = uint2;
  // Bytes of 8 codes (two's complement): each code offset by 128, an exact
  // integer in [1, 255], packed in place by the byte conversion, then the
  // offset's top bit flipped.
  __device__ static __forceinline__ Word encode8(const float* q) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(q[k] + 128.0f, k & 3, w[k >> 2]);
    return make_uint2(w[0] ^ 0x80808080u, w[1] ^ 0x80808080u);
  }
  __device__ static __forceinline__ int count_diff(Word x, Word y) {
    return bytes_differ(x.x ^ y.x) + bytes_differ(x.y ^ y.y);
  }
  __device__ static __forceinline__ void store8(uint8_t* dst, const float* q) {
    *reinterpret_cast<Word*>(dst) = encode8(q);
  }
};

// OCP E4M3FN elements. gfx950's FP8 conversion rounds a float32 to the
// nearest E4M3 value with ties to the even code (checked over every value,
// every midpoint and their float32 neighbours); magnitudes from just above
// 464 on become NaN, so inputs are clamped to +-456, which rounds to 448.
// A zero result keeps its sign (code 0x80), which storing clears.
template <> struct Grid<kGridE4M3> {
  static constexpr float qmax = 448.0f;
  static constexpr int kBits = 8;
  // Exact path: in binade [2^e, 2^(e+1)) (e >= -6; below that the subnormal
  // step) the values are k * 2^(e-3) with k in [8, 16), the code parity is
  // k's, and m*a is exact (m has at most 5 bits).
  __device__ static __forceinline__ float exact(float y, float w, float a, float b) {
    const float ay = __builtin_fminf(__builtin_fabsf(y), 456.0f);
    const int e = max(__builtin_amdgcn_frexp_expf(ay) - 1, -6);
    const float t = __builtin_ldexpf(ay, 3 - e);
    const float k = __builtin_floorf(t);
    const float m = __builtin_ldexpf(k + 0.5f, e - 3);
    const float d = __builtin_fmaf(-(m * a), b, __builtin_fabsf(w));
    const bool k_odd = ((int)k & 1) != 0;
    const float up = (d > 0.0f || (d == 0.0f && k_odd)) ? 1.0f : 0.0f;
    const float mag = __builtin_fminf(__builtin_ldexpf(k + up, e - 3), 448.0f);
    return __builtin_copysignf(mag, w);
  }
  // Four codes into one word (element p in byte p).
  __device__ static __forceinline__ uint32_t cvt4(const float* y) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
  }
  // Codes of N estimates by the same two-ended certificate as E2M1: the
  // exact quotient lies in [y (1 - 2^-20), y (1 + 2^-20)]; equal codes at
  // both ends are its codes. diff[g] receives the differing bytes of group
  // g of 4 elements (hiw is not used).
  template <int N>
  __device__ static __forceinline__ bool fast_n(const float* y, float* q, uint32_t* diff, uint32_t* hiw) {
    static_assert(N % 4 == 0, "groups of 4");
    uint32_t any = 0u;
#pragma unroll
    for (int g = 0; g < N; g += 4) {
      float lo[4], hi[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float yc = __builtin_amdgcn_fmed3f(y[g + k], -456.0f, 456.0f);
        lo[k] = yc * (1.0f - 0x1p-20f);
        hi[k] = yc * (1.0f + 0x1p-20f);
      }
      const uint32_t wl = cvt4(lo), wh = cvt4(hi);
      diff[g / 4] = wl ^ wh;
      any |= wl ^ wh;
      typedef float f2 __attribute__((ext_vector_type(2)));
      f2 r;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wl, 1.0f, false); q[g + 0] = r.x; q[g + 1] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wl, 1.0f, true);  q[g + 2] = r.x; q[g + 3] = r.y;
    }
    return any != 0u;
  }
  __device__ static __forceinline__ bool near(const float* y, const float* q, const uint32_t* diff,
                                              int e) {
    return ((diff[e >> 2] >> (8 * (e & 3))) & 0xFFu) != 0u;
  }
  // Rounded by two conversions; with eight levels per binade its ties are
  // more frequent than E2M1's and spread over more lanes, where testing each
  // slot with a vector compare is the cheaper re-decision (no kSlotMask).
  static constexpr bool kTwoEnded = true;
  static constexpr bool kSlotMask = false;
  static constexpr bool kScaledEnds = false;
  // Codes of N quotients that are exact: the conversion's own rounding is
  // the decision (magnitudes up to 456 saturate to 448).
  template <int N>
  __device__ static __forceinline__ void nearest_n(const float* y, float* q) {
    static_assert(N % 4 == 0, "groups of 4");
#pragma unroll
    for (int g = 0; g < N; g += 4) {
      float yc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) yc[k] = __builtin_amdgcn_fmed3f(y[g + k], -456.0f, 456.0f);
      const uint32_t w = cvt4(yc);
      typedef float f2 __attribute__((ext_vector_type(2)));
      f2 r;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false); q[g + 0] = r.x; q[g + 1] = r.y;
      r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);  q[g + 2] = r.x; q[g + 3] = r.y;
    }
  }
  // 8 codes as E4M3 bytes (exact values; a zero as +0), 8 bytes.
  using Word = uint2;
  __device__ static __forceinline__ Word encode8(const float* q) {
    uint32_t w[2] = {cvt4(q), cvt4(q + 4)};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t mag = w[i] & 0x7F7F7F7Fu;
      const uint32_t nonzero = (mag + 0x7F7F7F7Fu) & 0x80808080u;  // bit 7 set iff magnitude != 0
      w[i] &= 0x7F7F7F7Fu | nonzero;
    }
    return make_uint2(w[0], w[1]);
  }
  __device__ static __forceinline__ int count_diff(Word x, Word y) {
    return bytes_differ(x.x ^ y.x) + bytes_differ(x.y ^ y.y);
  }
  __device__ static __forceinline__ void store8(uint8_t* dst, const float* q) {
    *reinterpret_cast<Word*>(dst) = encode8(q);
  }
};

// ---------------------------------------------------------------- W loads

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Load 8 consecutive elements starting at p (16-byte aligned for bf16,
// 32 bytes = two 16-byte loads for float32) into float registers.
template <int WT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float* out) {
  if constexpr (WT == kWBF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    const float4 v0 = p[0], v1 = p[1];
    out[0] = v0.x; out[1] = v0.y; out[2] = v0.z; out[3] = v0.w;
    out[4] = v1.x; out[5] = v1.y; out[6] = v1.z; out[7] = v1.w;
  }
}

// One lane's LC contiguous elements of a row, as raw 16-byte vectors.
template <int WT, int LC> struct RawRow;

template <int LC> struct RawRow<kWBF16, LC> {
  uint4 v[LC / 8];
  __device__ __forceinline__ void load(const void* base, int64_t elem) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int i = 0; i < LC / 8; ++i) v[i] = p[i];
  }
  __device__ __forceinline__ void unpack(float* out) const {
#pragma unroll
    for (int i = 0; i < LC / 8; ++i) {
      out[8 * i + 0] = bf16_lo(v[i].x); out[8 * i + 1] = bf16_hi(v[i].x);
      out[8 * i + 2] = bf16_lo(v[i].y); out[8 * i + 3] = bf16_hi(v[i].y);
      out[8 * i + 4] = bf16_lo(v[i].z); out[8 * i + 5] = bf16_hi(v[i].z);
      out[8 * i + 6] = bf16_lo(v[i].w); out[8 * i + 7] = bf16_hi(v[i].w);
    }
  }
};

template <int LC> struct RawRow<kWF32, LC> {
  float4 v[LC / 4];
  __device__ __forceinline__ void load(const void* base, int64_t elem) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
#pragma unroll
    for (int i = 0; i < LC / 4; ++i) v[i] = p[i];
  }
  __device__ __forceinline__ void unpack(float* out) const {
#pragma unroll
    for (int i = 0; i < LC / 4; ++i) {
      out[4 * i + 0] = v[i].x; out[4 * i + 1] = v[i].y;
      out[4 * i + 2] = v[i].z; out[4 * i + 3] = v[i].w;
    }
  }
};

}  // namespace dq
