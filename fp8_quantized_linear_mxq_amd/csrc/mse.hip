// Weights with least-squared-error scales ("Bridging the Gap ... Microscaling
// FP4 Quantization" summary, MR-GPTQ modification 1: the grid is chosen for
// least MSE by optimising block scales and the tensor scale in turn).
//
// Block step: each block's scale code is the one, among every code of its
// scale format (E8M0 0..254 for MXFP4; E4M3 0..126 times g for NVFP4), whose
// squared error SSE = sum over the block's elements, in order, of
// (x - x_hat)^2 -- each subtraction, product and addition rounded to float64
// on its own -- is smallest, ties to the smaller code.  One lane owns one
// block and scans codes outward from the amax-rule code, which gives the
// exhaustive answer with few evaluations:
//  * upward, a code whose scale d has d / 4 >= amax rounds every element to
//    zero (SSE = sum x^2, which no code exceeds), and so does every larger
//    code: none of them can beat or tie-break ahead of a smaller code;
//  * downward, a code with 6 d < amax clips the largest element to 6 d, so
//    its SSE is at least that element's term (amax - 6 d)^2, which grows as
//    the code falls: once it exceeds the best SSE no smaller code can win.
// Tensor step (NVFP4): with block codes and element codes fixed, g = RN_fp32
// of P / Q, P = sum x w, Q = sum w^2 (w = element value times block scale),
// each a float64 sum of row sums in order; one thread per row, then one
// thread over the rows.  Rounds: amax-rule g, block step, tensor step, block
// step; MXFP4 runs one block step.
#include "device_common.h"
#include "kernels.h"

namespace mxq {
namespace {

constexpr int kThreads = 256;

struct MseP {
  const void* x;
  int64_t ldx;
  uint32_t bpr;        // blocks per row
  uint32_t nblk;       // rows * bpr
  uint8_t* codes;
  int64_t ld_codes;
  uint8_t* scales;
  int64_t ld_scales;
  const float* g;      // NVFP4 tensor scale (device)
  unsigned* dbg;
};

__device__ __forceinline__ double e2m1_mag(uint32_t c) {
  // magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6
  const uint32_t m = c & 7u;
  return m < 4u ? 0.5 * (double)m : (double)(2u << ((m - 4u) >> 1)) * ((m & 1u) ? 1.5 : 1.0);
}

template <int DT, int B>
__device__ __forceinline__ void load_block(const MseP& p, int64_t row, int64_t col, float (&v)[B]) {
  if constexpr (DT == DT_BF16) {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + row * p.ldx + col);
#pragma unroll
    for (int j = 0; j < B / 8; ++j) {
      const uint4 w = q[j];
      const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * j + 2 * i] = bf16_bits_to_f32(d[i] & 0xFFFFu);
        v[8 * j + 2 * i + 1] = bf16_bits_to_f32(d[i] >> 16);
      }
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p.x) + row * p.ldx + col);
#pragma unroll
    for (int j = 0; j < B / 4; ++j) {
      const float4 w = q[j];
      v[4 * j] = w.x; v[4 * j + 1] = w.y; v[4 * j + 2] = w.z; v[4 * j + 3] = w.w;
    }
  }
}

// Scale of candidate code c: 2**(c - 127) (MX) or E4M3(c) * g (NVFP4),
// exact in float64, and the element thresholds for it.
template <int FMT>
__device__ __forceinline__ double cand_scale(int c, float g, float th[7]) {
  if constexpr (FMT == FMT_MXFP4) {
    e2m1_thresholds_pow2(c - 127, th);
    return ldexp(1.0, c - 127);
  } else {
    const double d = (double)e4m3_value((uint32_t)c) * (double)g;
    e2m1_thresholds_f64(d, th);
    return d;
  }
}

// The block's SSE under scale d (thresholds th), in element order.
template <int B>
__device__ __forceinline__ double block_sse(const float (&v)[B], const float th[7], double d) {
#pragma clang fp contract(off)
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const uint32_t c = e2m1_encode(v[i], th);
    const double xh = (c & 8u) ? -(e2m1_mag(c) * d) : e2m1_mag(c) * d;
    const double diff = (double)v[i] - xh;
    s = s + diff * diff;
  }
  return s;
}

// Block step: one lane per block (32 for MXFP4, 16 for NVFP4); FINAL also
// writes the element codes under the chosen scale.
template <int DT, int FMT, bool FINAL>
__global__ __launch_bounds__(kThreads) void mse_block_kernel(MseP p) {
#pragma clang fp contract(off)
  constexpr int B = FMT == FMT_NVFP4 ? 16 : 32;
  constexpr int CMAX = FMT == FMT_NVFP4 ? 126 : 254;
  float g = 0.f;
  if constexpr (FMT == FMT_NVFP4) g = *p.g;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < p.nblk; b += gridDim.x * kThreads) {
    const int64_t row = b / p.bpr, col = (int64_t)(b - (uint32_t)row * p.bpr) * B;
    float v[B];
    load_block<DT, B>(p, row, col, v);
    if (p.dbg) {
      bool bad = false;
#pragma unroll
      for (int i = 0; i < B; ++i) bad |= !__builtin_isfinite(v[i]);
      if (bad) atomicOr(p.dbg, 1u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < B; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // the amax rule's code
    int c0;
    if constexpr (FMT == FMT_MXFP4) c0 = mx_exponent(amax, 2) + 127;
    else c0 = (g == 0.f) ? 0 : (int)e4m3_encode_f64((double)amax / (6.0 * (double)g));
    float th[7];
    double best = block_sse<B>(v, th, cand_scale<FMT>(c0, g, th));
    int bc = c0;
    // upward until every element rounds to zero
    for (int c = c0 + 1; c <= CMAX; ++c) {
      const double d = cand_scale<FMT>(c, g, th);
      if (0.25 * d >= (double)amax) break;
      const double sse = block_sse<B>(v, th, d);
      if (sse < best) { best = sse; bc = c; }
    }
    // downward until the clipped largest element alone outweighs the best
    for (int c = c0 - 1; c >= 0; --c) {
      const double d = cand_scale<FMT>(c, g, th);
      if (6.0 * d < (double)amax) {
        const double clip = (double)amax - 6.0 * d;
        if (clip * clip > best) break;
      }
      const double sse = block_sse<B>(v, th, d);
      if (sse <= best) { best = sse; bc = c; }   // ties go to the smaller code
    }
    p.scales[row * p.ld_scales + col / B] = (uint8_t)bc;
    if constexpr (FINAL) {
      cand_scale<FMT>(bc, g, th);
      uint32_t w[B / 8];
#pragma unroll
      for (int j = 0; j < B / 8; ++j) {
        w[j] = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w[j] |= e2m1_encode(v[8 * j + i], th) << (4 * i);
      }
      uint8_t* dst = p.codes + row * p.ld_codes + col / 2;
      if constexpr (B == 32) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      else *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    }
  }
}

// Tensor step, per row: P_r = sum x w, Q_r = sum w w over the row in order
// (w = +-E2M1 value times the block's E4M3 value under scale v * g0; x w and
// w w are exact in float64, the additions round).
template <int DT>
__global__ __launch_bounds__(64) void mse_rows_kernel(MseP p, int64_t rows, double* pq) {
#pragma clang fp contract(off)
  const int64_t row = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (row >= rows) return;
  const float g = *p.g;
  double sp = 0.0, sq = 0.0;
  for (uint32_t blk = 0; blk < p.bpr; ++blk) {
    float v[16];
    load_block<DT, 16>(p, row, (int64_t)blk * 16, v);
    const uint32_t sc = p.scales[row * p.ld_scales + blk];
    const double sv = (double)e4m3_value(sc);
    float th[7];
    e2m1_thresholds_f64(sv * (double)g, th);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = e2m1_encode(v[i], th);
      const double w = (c & 8u) ? -(e2m1_mag(c) * sv) : e2m1_mag(c) * sv;
      sp = sp + (double)v[i] * w;
      sq = sq + w * w;
    }
  }
  pq[2 * row] = sp;
  pq[2 * row + 1] = sq;
}

// Tensor step, over the rows in order: g1 = RN_fp32(P / Q); Q = 0 or a
// quotient that rounds to 0 keeps g0.
__global__ __launch_bounds__(64) void mse_tensor_kernel(const double* pq, int64_t rows,
                                                        const float* g0, float* g_out) {
#pragma clang fp contract(off)
  if (threadIdx.x != 0) return;
  double P = 0.0, Q = 0.0;
  for (int64_t r = 0; r < rows; ++r) {
    P = P + pq[2 * r];
    Q = Q + pq[2 * r + 1];
  }
  float g = *g0;
  if (Q != 0.0) {
    const float g1 = (float)(P / Q);
    if (g1 != 0.f) g = g1;
  }
  *g_out = g;
}

template <int DT>
hipError_t launch_dt(const MseArgs& a, hipStream_t s) {
  MseP p;
  p.x = a.x;
  p.ldx = a.ldx;
  p.codes = a.codes;
  p.ld_codes = a.ld_codes;
  p.scales = a.scales;
  p.ld_scales = a.ld_scales;
  p.dbg = a.dbg;
  p.g = nullptr;
  const int B = a.fmt == FMT_NVFP4 ? 16 : 32;
  p.bpr = (uint32_t)(a.cols / B);
  p.nblk = (uint32_t)(a.rows * p.bpr);
  uint32_t blocks = (p.nblk + kThreads - 1) / kThreads;
  if (blocks > 8192u) blocks = 8192u;
  if (a.fmt == FMT_MXFP4) {
    mse_block_kernel<DT, FMT_MXFP4, true><<<blocks, kThreads, 0, s>>>(p);
    return hipGetLastError();
  }
  char* ws = static_cast<char*>(a.ws);
  float* partials = reinterpret_cast<float*>(ws);
  float* g0 = reinterpret_cast<float*>(ws + (size_t)kAmaxPartials * 4);
  double* pq = reinterpret_cast<double*>(ws + (size_t)kAmaxPartials * 4 + 16);
  hipError_t e = launch_nvfp4_tensor_scale(a.x, a.dtype, a.rows, a.cols, a.ldx, partials, g0,
                                           nullptr, s);
  if (e != hipSuccess) return e;
  p.g = g0;
  mse_block_kernel<DT, FMT_NVFP4, false><<<blocks, kThreads, 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  mse_rows_kernel<DT><<<(unsigned)((a.rows + 63) / 64), 64, 0, s>>>(p, a.rows, pq);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  mse_tensor_kernel<<<1, 64, 0, s>>>(pq, a.rows, g0, a.tensor_scale_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.g = a.tensor_scale_out;
  mse_block_kernel<DT, FMT_NVFP4, true><<<blocks, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

int64_t mse_workspace_bytes(int fmt, int64_t rows) {
  return fmt == FMT_NVFP4 ? (int64_t)kAmaxPartials * 4 + 16 + rows * 16 : 0;
}

hipError_t launch_quantize_mse(const MseArgs& a, hipStream_t s) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  return a.dtype == DT_BF16 ? launch_dt<DT_BF16>(a, s) : launch_dt<DT_F32>(a, s);
}

}  // namespace mxq
