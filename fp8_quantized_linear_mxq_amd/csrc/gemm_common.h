// Pieces shared by the GEMM routes: parameters, tile order, LDS swizzle and
// the epilogue (low-rank branch, bias, bf16 rounding, column map).
#pragma once

#include "device_common.h"

namespace mxq {

constexpr int BM = 128, BN = 128;
constexpr int kThreads = 256;

// XOR swizzle of 16-byte chunks within an LDS row of CH chunks: a wave's
// 16-byte fragment reads (one row per lane) then hit distinct banks.
template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 2) return (r >> 2) & 1;
  else if constexpr (CH == 4) return ((r >> 2) ^ (r & 2)) & 3;
  else return ((r >> 1) ^ ((r & 1) << 2)) & 7;
}

struct GemmP {
  const uint8_t* a; int64_t lda; const uint8_t* as; int64_t ldas;
  const uint8_t* w; int64_t ldw; const uint8_t* ws; int64_t ldws;
  int M, N, K;
  int tiles_m, tiles_n;
  const int32_t* col_map;
  const float* u; int64_t ld_u; const uint16_t* l2t; int rank;
  const uint16_t* bias;
  uint16_t* out; int64_t ld_out; int n_out;
  // Implicit im2col of a 3x3, stride-1, zero-padded convolution when cv_c > 0:
  // A's codes and scales are the input's [images * cv_h * cv_w][cv_c] pixel
  // rows; GEMM row m is output pixel m (row-major image, y, x) and K index
  // (ky*3 + kx)*cv_c + c reads channel c of input pixel (y + ky - 1,
  // x + kx - 1), zero outside the image.  cv_c is a multiple of the K-tile,
  // so a K-tile never spans two taps.
  int cv_h, cv_w, cv_c;
};

// K-tiles per tap (cv_c / bk) and ceil(2**32 / tiles): floor(kt / tiles) is
// then one multiply, exact while kt * tiles < 2**32, which holds for every
// K-tile when cv_c <= 2**20 (kt < 9 * tiles, tiles <= 2**14).
struct ConvDiv {
  uint32_t tiles;
  uint64_t magic;
};

__device__ __forceinline__ ConvDiv conv_div(const GemmP& p, int bk) {
  ConvDiv d;
  d.tiles = (uint32_t)(p.cv_c / bk);
  d.magic = ((1ull << 32) + d.tiles - 1) / d.tiles;
  return d;
}

// The tap (ky * 3 + kx) of K-tile kt of an implicit-im2col operand, its
// pixel offsets (dy, dx) = (ky - 1, kx - 1), the K-tile's index inside the
// channel row, and the row shift dy * width + dx.
struct ConvTap {
  int tap, dy, dx, kc, shift;
};

__device__ __forceinline__ ConvTap conv_tap(const GemmP& p, const ConvDiv& d, int kt) {
  ConvTap t;
  t.tap = (int)(((uint64_t)(uint32_t)kt * d.magic) >> 32);
  t.kc = kt - t.tap * (int)d.tiles;
  t.dy = t.tap / 3 - 1;
  t.dx = t.tap - 3 * (t.tap / 3) - 1;
  t.shift = t.dy * p.cv_w + t.dx;
  return t;
}

// Bit t of the mask is set when tap t of GEMM row `row` reads a pixel inside
// the image (computed once per row; a K-tile then tests one bit).
__device__ __forceinline__ uint32_t conv_mask(const GemmP& p, int row) {
  const int hw = row % (p.cv_h * p.cv_w);
  const int y = hw / p.cv_w, x = hw - (hw / p.cv_w) * p.cv_w;
  uint32_t m = 0;
#pragma unroll
  for (int t = 0; t < 9; ++t) {
    const int yy = y + t / 3 - 1, xx = x + t % 3 - 1;
    m |= ((unsigned)yy < (unsigned)p.cv_h && (unsigned)xx < (unsigned)p.cv_w) ? (1u << t) : 0u;
  }
  return m;
}

__device__ __forceinline__ bool conv_inside(uint32_t mask, const ConvTap& t) {
  return (mask >> t.tap) & 1u;
}

__device__ __forceinline__ int remap_tile(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = bid & 7, y = bid >> 3;
  return x < r ? x * (q + 1) + y : r * (q + 1) + (x - r) * q + y;
}

template <int OPSEL, int AF>
__device__ __forceinline__ v16f mfma_scaled(const v8i& a, const v8i& b, const v16f& c, int sa,
                                            int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, AF, 4, OPSEL, sa, OPSEL, sb);
}

// Epilogue shared with the other routes: add the low-rank branch on the
// bf16 MFMA, bias, convert and store through the optional column map.
template <bool LR>
__device__ __forceinline__ void epilogue(const GemmP& p, v16f acc[2][2], float alpha,
                                         int m0, int n0, int wm, int wn, int lane) {
  const int l32 = lane & 31, half = lane >> 5;
  int col_out[2];
  bool col_ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + l32;
    int c = -1;
    if (n < p.N) c = p.col_map ? p.col_map[n] : n;
    col_ok[j] = (c >= 0 && c < p.n_out);
    col_out[j] = col_ok[j] ? c : 0;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] *= alpha;

  if constexpr (LR) {
    // u = u_hi + u_lo (bf16 halves, residual <= 2**-18 |u|) times L2 on the
    // bf16 MFMA, K = rank for each half.
    for (int t = 0; t < p.rank / 16; ++t) {
      v8bf bfrag[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(
            p.l2t + (int64_t)col_out[j] * p.rank + t * 16 + half * 8);
        bfrag[j] = __builtin_bit_cast(v8bf, v);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int row = m0 + wm * 64 + i * 32 + l32;
        row = row < p.M ? row : p.M - 1;
        const float* up = p.u + (int64_t)row * p.ld_u + t * 16 + half * 8;
        const float4 f0 = *reinterpret_cast<const float4*>(up);
        const float4 f1 = *reinterpret_cast<const float4*>(up + 4);
        const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          hi[e] = f32_to_bf16_bits(f[e]);
          lo[e] = f32_to_bf16_bits(f[e] - bf16_bits_to_f32(hi[e]));
        }
        uint4 hv, lv;
        hv.x = hi[0] | (hi[1] << 16); hv.y = hi[2] | (hi[3] << 16);
        hv.z = hi[4] | (hi[5] << 16); hv.w = hi[6] | (hi[7] << 16);
        lv.x = lo[0] | (lo[1] << 16); lv.y = lo[2] | (lo[3] << 16);
        lv.z = lo[4] | (lo[5] << 16); lv.w = lo[6] | (lo[7] << 16);
        const v8bf ah = __builtin_bit_cast(v8bf, hv), al = __builtin_bit_cast(v8bf, lv);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bfrag[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bfrag[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float b = (p.bias && col_ok[j]) ? bf16_bits_to_f32(p.bias[col_out[j]]) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
        if (row < p.M && col_ok[j])
          __builtin_nontemporal_store((uint16_t)f32_to_bf16_bits(acc[i][j][q] + b),
                                      &p.out[(int64_t)row * p.ld_out + col_out[j]]);
      }
    }
  }
}

namespace {

// Split-K finish: y = RN_bf16(alpha * sum over splits (in split order) +
// bias), stored through the column map; part is [splits][M][N] fp32.  One
// thread per output element.  (A copy per translation unit.)
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const float* part, int splits,
                                                               int M, int N, const float* a_gp,
                                                               float pow2,
                                                               const int32_t* col_map,
                                                               const uint16_t* bias,
                                                               uint16_t* out, int64_t ld_out,
                                                               int n_out) {
  // pow2: the power of two undoing the activations' dequantization bias
  const float alpha = a_gp ? pow2 * *a_gp : pow2;
  const int64_t total = (int64_t)M * N;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int row = (int)(e / N), n = (int)(e % N);
    const int c = col_map ? col_map[n] : n;
    if (c < 0 || c >= n_out) continue;
    float sum = 0.f;
    for (int sp = 0; sp < splits; ++sp) sum += part[(int64_t)sp * total + e];
    const float v = alpha * sum + (bias ? bf16_bits_to_f32(bias[c]) : 0.f);
    out[(int64_t)row * ld_out + c] = (uint16_t)f32_to_bf16_bits(v);
  }
}

inline hipError_t launch_splitk_reduce(const GemmP& g, const float* part, int splits,
                                       const float* alpha, float pow2, hipStream_t s) {
  const int64_t total = (int64_t)g.M * g.N;
  const int64_t want = (total + kThreads - 1) / kThreads;
  const int blocks = (int)(want < 4096 ? want : 4096);
  splitk_reduce_kernel<<<blocks, kThreads, 0, s>>>(part, splits, g.M, g.N, alpha, pow2, g.col_map,
                                                   g.bias, g.out, g.ld_out, g.n_out);
  return hipGetLastError();
}

}  // namespace

}  // namespace mxq
