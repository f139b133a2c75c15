// Device helpers shared by the libmxq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Format identifiers (same values as mxq_format in mxq.h).
enum : int { FMT_MXFP4 = 1, FMT_MXFP8 = 2, FMT_NVFP4 = 3, FMT_INT4 = 4, FMT_BF16 = 5 };
enum : int { DT_F32 = 1, DT_BF16 = 2 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float next_up_pos(float f) {  // f >= 0, finite
  return __uint_as_float(__float_as_uint(f) + 1u);
}

// Lane exchange with lane ^ M inside a wave64.
template <int M>
__device__ __forceinline__ int xor_lane(int v) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (M < 32) {
    return __builtin_amdgcn_ds_swizzle(v, 0x1F | (M << 10));    // bitmask mode, xor M
  } else {
    return __shfl_xor(v, M);
  }
}

template <int M>
__device__ __forceinline__ float xor_lane_f(float v) {
  return __int_as_float(xor_lane<M>(__float_as_int(v)));
}

template <int M>
__device__ __forceinline__ double xor_lane_d(double v) {
  int2 p = *reinterpret_cast<int2*>(&v);
  p.x = xor_lane<M>(p.x);
  p.y = xor_lane<M>(p.y);
  return *reinterpret_cast<double*>(&p);
}

// Max over a group of G consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 2) v = fmaxf(v, xor_lane_f<1>(v));
  if constexpr (G >= 4) v = fmaxf(v, xor_lane_f<2>(v));
  if constexpr (G >= 8) v = fmaxf(v, xor_lane_f<4>(v));
  if constexpr (G >= 16) v = fmaxf(v, xor_lane_f<8>(v));
  if constexpr (G >= 32) v = fmaxf(v, xor_lane_f<16>(v));
  if constexpr (G >= 64) v = fmaxf(v, xor_lane_f<32>(v));
  return v;
}

// ---------------------------------------------------------------------------
// Element encoders.  Every one decides on the exact real value.
// ---------------------------------------------------------------------------

// E2M1 by thresholds: code magnitude = number of u[i] <= |x|, where u[i] is
// the smallest float32 that rounds up across the i-th midpoint (see
// e2m1_thresholds_*).  The sign bit copies the sign of x.
__device__ __forceinline__ uint32_t e2m1_encode(float x, const float u[7]) {
  float a = fabsf(x);
  uint32_t c = (uint32_t)(a >= u[0]) + (uint32_t)(a >= u[1]) + (uint32_t)(a >= u[2]) +
               (uint32_t)(a >= u[3]) + (uint32_t)(a >= u[4]) + (uint32_t)(a >= u[5]) +
               (uint32_t)(a >= u[6]);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// E2M1 midpoints between consecutive magnitudes 0,.5,1,1.5,2,3,4,6.  A tie at
// an even index rounds down (to the even code), at an odd index up.
__device__ __forceinline__ void e2m1_thresholds_pow2(int e, float u[7]) {
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    float t = ldexpf(mids[i], e);          // exact (power-of-two scale)
    u[i] = (i & 1) ? t : next_up_pos(t);   // odd: >= t counts; even: > t counts
  }
}

// Thresholds for the scale d = s * g (exact in float64).  t = mid * d is exact
// in float64; u is the smallest float32 >= t (odd) or > t (even).  d == 0
// makes every element a signed zero.
__device__ __forceinline__ void e2m1_thresholds_f64(double d, float u[7]) {
  const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  if (d == 0.0) {
#pragma unroll
    for (int i = 0; i < 7; ++i) u[i] = __builtin_inff();
    return;
  }
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    double t = mids[i] * d;
    float f = (float)t;                    // nearest float32
    if ((double)f < t) f = next_up_pos(f); // now the smallest float32 >= t
    if (!(i & 1) && (double)f == t) f = next_up_pos(f);
    u[i] = f;
  }
}

// The same thresholds for d = s * g (s an E4M3 value, g a positive fp32)
// without float64 products.  d = d_hi + d_lo exactly (fma residual; s has 4
// significant bits, so d_lo is short); t = mid * d = t_hi + e with t_hi the
// rounded mid * d_hi and e = (fma residual of mid * d_hi) + mid * d_lo, both
// terms short and close in scale, so e is exact.  u = RN(t_hi + e) is the
// float32 nearest t and r = e - (u - t_hi) the exact remainder t - u
// (Fast2Sum, |t_hi| >= |e|), |r| <= half an ulp of u: the smallest float32
// >= t (odd i) is u unless r > 0, the smallest > t (even i) u unless r >= 0.
// Valid while every residual is a normal float32; smaller d (below 2**-60)
// takes the float64 path.  Every product and sum here must round on its own:
// a multiply fused into a later add (t_hi into n or into n - t_hi) breaks the
// error-free steps, so contraction is off in this function.
__device__ __forceinline__ void e2m1_thresholds_sg(float s, float g, float u[7]) {
#pragma clang fp contract(off)
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  const float d_hi = s * g;
  if (!(d_hi >= 0x1p-60f)) {          // zero, or close enough to underflow
    e2m1_thresholds_f64((double)s * (double)g, u);
    return;
  }
  const float d_lo = __builtin_fmaf(s, g, -d_hi);
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    const float t_hi = mids[i] * d_hi;
    const float e = __builtin_fmaf(mids[i], d_hi, -t_hi) + mids[i] * d_lo;
    const float n = t_hi + e;
    const float r = e - (n - t_hi);
    const bool up = (i & 1) ? (r > 0.f) : (r >= 0.f);
    u[i] = up ? next_up_pos(n) : n;
  }
}

// E4M3 (OCP FN: bias 7, max 448, no Inf) of an exactly scaled value v with
// |v| < 512, nearest-even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {                     // below 2**-6: subnormal quantum 2**-9
    code = (uint32_t)rintf(a * 512.0f);    // 0..8; 8 is the code of 2**-6
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);      // round mantissa to 3 bits, ties even
    uint32_t ex = (b >> 23) - 120u;        // (exp - 127) + 7
    code = (ex << 3) | ((b >> 20) & 7u);
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code | ((__float_as_uint(v) >> 24) & 0x80u);
}

// E4M3 of a non-negative float64 value, nearest-even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode_f64(double a) {
  if (a < 0.015625) return (uint32_t)rint(a * 512.0);
  if (a >= 464.0) return 0x7Eu;            // 464 ties 448|480 -> 448; above saturates
  uint64_t b = (uint64_t)__double_as_longlong(a);
  b += 0x0000FFFFFFFFFFFFull + ((b >> 49) & 1ull);   // round 52 -> 3 mantissa bits
  uint32_t ex = (uint32_t)(b >> 52) - 1016u;          // (exp - 1023) + 7
  uint32_t code = (ex << 3) | (uint32_t)((b >> 49) & 7ull);
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {  // positive codes
  uint32_t ex = (code >> 3) & 15u, m = code & 7u;
  if (ex == 0) return (float)m * 0.001953125f;               // m * 2**-9
  return __uint_as_float(((ex + 120u) << 23) | (m << 20));
}

// MX shared exponent from the block amax: floor(log2 amax) - emax, clamped.
__device__ __forceinline__ int mx_exponent(float amax, int emax) {
  int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  int e = E - 127 - emax;
  return (E == 0 || e < -127) ? -127 : e;
}

}  // namespace mxq
