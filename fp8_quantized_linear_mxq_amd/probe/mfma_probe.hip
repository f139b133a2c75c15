// Matrix-core probes for the design notes (not part of libmxq; built as its
// own shared library, libmxq_probe.so, by build.py):
//  * probe_mfma_rate: how fast the gfx950 matrix cores run a stream of
//    independent MFMAs from registers, with random or all-zero operands (the
//    clock drops under the switching power of random data), for the MFMA
//    kinds the GEMM routes use;
//  * probe_mfma_sum: one MFMA of a given kind on caller-given operands and
//    per-lane block scales, so that the host can compare every output with
//    the exact sum of its products;
//  * probe_cvt_scale: the scaled E2M1 converts with arbitrary fp32 scales
//    (whether a non-power-of-two scale is applied exactly).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {

constexpr int NACC = 8;   // independent accumulators per wave

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  return x;
}

// KIND 0: scaled E2M1 x E2M1 32x32x64; 1: scaled E4M3 x E2M1 32x32x64;
// 2: bf16 32x32x16.
template <int KIND>
__global__ __launch_bounds__(512) void mfma_rate_kernel(int iters, int zero, float* out) {
  const uint32_t seed = (blockIdx.x * blockDim.x + threadIdx.x) * 0x9E3779B9u;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = zero ? 0 : (int)hash32(seed + i);
    b[i] = zero ? 0 : (int)hash32(seed + 100 + i);
  }
  if (KIND == 1) {   // E4M3 bytes with exponent field <= 13: no NaN codes
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] &= (int)0xEFEFEFEFu;
  }
  if (KIND == 2) {   // bf16 halves with exponent field < 128: finite
#pragma unroll
    for (int i = 0; i < 8; ++i) { a[i] &= (int)0xBFFFBFFFu; b[i] &= (int)0xBFFFBFFFu; }
  }
  v16f acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = v16f{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NACC; ++j) {
      if constexpr (KIND == 0)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 4, 4, 0, 127, 0, 127);
      else if constexpr (KIND == 1)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 4, 0, 127, 0, 127);
      else
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(v8bf, __builtin_shufflevector(a, a, 0, 1, 2, 3)),
            __builtin_bit_cast(v8bf, __builtin_shufflevector(b, b, 0, 1, 2, 3)), acc[j], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) s += acc[j][q];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// One wave, one MFMA from a zero accumulator.  Operand lane layout (all
// kinds): lane l carries row l % 32 of its matrix; the two lane halves carry
// the two halves of K.  a_ops / b_ops: 8 dwords per lane (kinds 0-2 use 8
// E4M3 or 4 E2M1 dwords, kind 3 two E4M3 dwords, kind 4 four bf16 dwords);
// a_scl / b_scl: one E8M0 code per lane (scaled kinds).
//   KIND 0: scaled E4M3 x E2M1 32x32x64    1: scaled E2M1 x E2M1 32x32x64
//        2: scaled E4M3 x E4M3 32x32x64    3: E4M3 x E4M3 32x32x16
//        4: bf16 x bf16 32x32x16
template <int KIND>
__global__ __launch_bounds__(64) void mfma_sum_kernel(const int* a_ops, const int* b_ops,
                                                      const int* a_scl, const int* b_scl, float* d) {
  const int l = threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) { a[i] = a_ops[l * 8 + i]; b[i] = b_ops[l * 8 + i]; }
  const int sa = a_scl[l], sb = b_scl[l];
  v16f acc = v16f{};
  if constexpr (KIND == 0)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 4, 0, sa, 0, sb);
  else if constexpr (KIND == 1)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 4, 4, 0, sa, 0, sb);
  else if constexpr (KIND == 2)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb);
  else if constexpr (KIND == 3) {
    const long al = (long)(uint32_t)a[0] | ((long)a[1] << 32);
    const long bl = (long)(uint32_t)b[0] | ((long)b[1] << 32);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(al, bl, acc, 0, 0, 0);
  } else
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(v8bf, __builtin_shufflevector(a, a, 0, 1, 2, 3)),
        __builtin_bit_cast(v8bf, __builtin_shufflevector(b, b, 0, 1, 2, 3)), acc, 0, 0, 0);
#pragma unroll
  for (int q = 0; q < 16; ++q) d[l * 16 + q] = acc[q];
}

// Thread i converts all 16 E2M1 codes with scale scales[i] through one of
// the scaled converts (KIND 0: pk_f16_fp4, 1: pk_bf16_fp4, 2: pk_f32_fp4)
// and writes the 16 results' bits (16-bit results zero-extended) to
// out[16 i .. 16 i + 15].
template <int KIND, int SEL>
__device__ __forceinline__ void cvt_pair(uint32_t word, float s, uint32_t& lo, uint32_t& hi) {
  typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
  typedef __bf16 v2b_t __attribute__((ext_vector_type(2)));
  typedef float v2f_t __attribute__((ext_vector_type(2)));
  if constexpr (KIND == 0) {
    const v2h_t r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, s, SEL);
    lo = __builtin_bit_cast(uint16_t, r.x); hi = __builtin_bit_cast(uint16_t, r.y);
  } else if constexpr (KIND == 1) {
    const v2b_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, SEL);
    lo = __builtin_bit_cast(uint16_t, r.x); hi = __builtin_bit_cast(uint16_t, r.y);
  } else {
    const v2f_t r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, s, SEL);
    lo = __float_as_uint(r.x); hi = __float_as_uint(r.y);
  }
}

// Thread i converts all 16 E2M1 codes with scale scales[i] through one of
// the scaled converts (KIND 0: pk_f16_fp4, 1: pk_bf16_fp4, 2: pk_f32_fp4)
// and writes the 16 results' bits (16-bit results zero-extended) to
// out[16 i .. 16 i + 15].
template <int KIND>
__global__ __launch_bounds__(256) void cvt_scale_kernel(const float* scales, int n, uint32_t* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float s = scales[i];
  const uint32_t words[2] = {0x76543210u, 0xFEDCBA98u};
  uint32_t r[16];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    cvt_pair<KIND, 0>(words[w], s, r[8 * w + 0], r[8 * w + 1]);
    cvt_pair<KIND, 1>(words[w], s, r[8 * w + 2], r[8 * w + 3]);
    cvt_pair<KIND, 2>(words[w], s, r[8 * w + 4], r[8 * w + 5]);
    cvt_pair<KIND, 3>(words[w], s, r[8 * w + 6], r[8 * w + 7]);
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) out[16 * i + k] = r[k];
}

}  // namespace

extern "C" {

// The scaled E2M1 converts on every code for n caller-given fp32 scales
// (device pointers; out: n * 16 uint32).  kind 0: to f16, 1: to bf16,
// 2: to f32.  Returns a hipError_t.
int probe_cvt_scale(int kind, const float* scales, int n, uint32_t* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!scales || !out || n < 1) return (int)hipErrorInvalidValue;
  const dim3 g((n + 255) / 256), t(256);
  if (kind == 0) cvt_scale_kernel<0><<<g, t, 0, s>>>(scales, n, out);
  else if (kind == 1) cvt_scale_kernel<1><<<g, t, 0, s>>>(scales, n, out);
  else if (kind == 2) cvt_scale_kernel<2><<<g, t, 0, s>>>(scales, n, out);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// Enqueues `blocks` workgroups of `waves` waves, each wave issuing
// iters * 8 independent MFMAs of `kind` (0 FP4 scaled, 1 FP8 x FP4 scaled,
// 2 bf16); out: device, blocks * waves * 64 floats.  Returns a hipError_t.
int probe_mfma_rate(int kind, int blocks, int waves, int iters, int zero, float* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (waves < 1 || waves > 8 || blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
  const dim3 g(blocks), t(64 * waves);
  if (kind == 0) mfma_rate_kernel<0><<<g, t, 0, s>>>(iters, zero, out);
  else if (kind == 1) mfma_rate_kernel<1><<<g, t, 0, s>>>(iters, zero, out);
  else if (kind == 2) mfma_rate_kernel<2><<<g, t, 0, s>>>(iters, zero, out);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// One MFMA of `kind` (0-4, see mfma_sum_kernel).  Device pointers: a_ops,
// b_ops 64 x 8 ints; a_scl, b_scl 64 ints; d 64 x 16 floats, lane l's
// accumulator registers in order.  Returns a hipError_t.
int probe_mfma_sum(int kind, const int* a_ops, const int* b_ops, const int* a_scl, const int* b_scl,
                   float* d, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!a_ops || !b_ops || !a_scl || !b_scl || !d) return (int)hipErrorInvalidValue;
  switch (kind) {
    case 0: mfma_sum_kernel<0><<<1, 64, 0, s>>>(a_ops, b_ops, a_scl, b_scl, d); break;
    case 1: mfma_sum_kernel<1><<<1, 64, 0, s>>>(a_ops, b_ops, a_scl, b_scl, d); break;
    case 2: mfma_sum_kernel<2><<<1, 64, 0, s>>>(a_ops, b_ops, a_scl, b_scl, d); break;
    case 3: mfma_sum_kernel<3><<<1, 64, 0, s>>>(a_ops, b_ops, a_scl, b_scl, d); break;
    case 4: mfma_sum_kernel<4><<<1, 64, 0, s>>>(a_ops, b_ops, a_scl, b_scl, d); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}
