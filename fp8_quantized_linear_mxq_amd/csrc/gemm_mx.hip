// Block-scaled GEMM on the gfx950 scaled MFMA: y = RN_bf16(Q(a) Q(w)^T [+ u L2] [+ bias]).
//
// The 4-bit weight x 4-bit activation product is the layer's one dense
// contraction (Nunchaku article, "main explanation": W4A4 speeds up the
// denoising loop; the 16-bit low-rank branch is added to the same output).
// v_mfma_scale_f32_32x32x64_f8f6f4 consumes E2M1 codes directly and applies
// one E8M0 scale per lane per 32 K-values, which is exactly the MX block
// (Microscaling FP4 summary: power-of-two MXFP4 scales), so codes and scales
// go from HBM to the matrix core with no conversion.  For E2M1 x E2M1 its
// dot products are exact before the fp32 accumulation (measured); with E4M3
// operands they are not, so MXFP8 activations take the dequantizing route.
// The kernel keeps the E4M3 operand path (AF = 0) for completeness.
//
// Operand layouts (checked on gfx950): lane l of a 32x32x64 step holds row
// l % 32; for E2M1 its 32 codes are K = 32*(l/32) + [0,32); for E4M3 they are
// split 16 + 16 (see the A-fragment load).  Either way the lane's scale
// register supplies the E8M0 of K-block l/32 of its row.
//
// Tiling: 128x128 output tile per 256-thread workgroup, 2x2 waves of 64x64,
// each wave 2x2 MFMA tiles of 32x32; K-tile 128 (two MFMA K-steps of 64).
// Codes are staged through double-buffered LDS with a 16-byte-chunk XOR
// swizzle; the per-row scale bytes of a K-tile (4 blocks) are one dword
// loaded straight into registers, and the MFMA op_sel picks the byte.
// Workgroup ids are remapped so each XCD works on a contiguous tile range.
#include "device_common.h"
#include "kernels.h"
#include "gemm_common.h"

namespace mxq {
namespace {

constexpr int BK = 128;
constexpr int kSlabTiles = 16;   // K-tiles (2 MFMA steps each) per fp32 slab

// AF: MFMA format code of the activation codes (0 = E4M3, 4 = E2M1).
template <int AF, bool LR, bool SLAB>
__global__ __launch_bounds__(kThreads) void gemm_mx_kernel(GemmP p) {
  constexpr int A_RB = (AF == 4) ? 64 : 128;  // bytes per row per K-tile
  constexpr int B_RB = 64;
  constexpr int A_CH = A_RB / 16, B_CH = B_RB / 16;
  constexpr int A_LOADS = BM * A_CH / kThreads, B_LOADS = BN * B_CH / kThreads;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * A_RB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * B_RB];

  const int tile = remap_tile(blockIdx.x, p.tiles_m * p.tiles_n);
  const int m0 = (tile / p.tiles_n) * BM, n0 = (tile % p.tiles_n) * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, half = lane >> 5;
  const int KT = p.K / BK;

  // global -> LDS chunk assignment
  const uint8_t* ga[A_LOADS];
  int la[A_LOADS];
  bool va[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int q = tid + i * kThreads, r = q / A_CH, c = q % A_CH;
    va[i] = (m0 + r) < p.M;
    ga[i] = p.a + (int64_t)(va[i] ? m0 + r : 0) * p.lda + c * 16;
    la[i] = r * A_RB + ((c ^ swz<A_CH>(r)) * 16);
  }
  const uint8_t* gb[B_LOADS];
  int lb[B_LOADS];
  bool vb[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int q = tid + i * kThreads, r = q / B_CH, c = q % B_CH;
    vb[i] = (n0 + r) < p.N;
    gb[i] = p.w + (int64_t)(vb[i] ? n0 + r : 0) * p.ldw + c * 16;
    lb[i] = r * B_RB + ((c ^ swz<B_CH>(r)) * 16);
  }
  // scale rows for this lane's MFMA fragments (clamped; results discarded)
  const uint8_t* sa_row[2];
  const uint8_t* sb_row[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int r = m0 + wm * 64 + i * 32 + l32;
    sa_row[i] = p.as + (int64_t)(r < p.M ? r : p.M - 1) * p.ldas;
    int c = n0 + wn * 64 + i * 32 + l32;
    sb_row[i] = p.ws + (int64_t)(c < p.N ? c : p.N - 1) * p.ldws;
  }

  uint4 ra[A_LOADS], rb[B_LOADS];
  uint32_t sa[2], sb[2], nsa[2], nsb[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      ra[i] = va[i] ? *reinterpret_cast<const uint4*>(ga[i] + (int64_t)kt * A_RB)
                    : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      rb[i] = vb[i] ? *reinterpret_cast<const uint4*>(gb[i] + (int64_t)kt * B_RB)
                    : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      nsa[i] = *reinterpret_cast<const uint32_t*>(sa_row[i] + kt * 4) >> (8 * half);
      nsb[i] = *reinterpret_cast<const uint32_t*>(sb_row[i] + kt * 4) >> (8 * half);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) *reinterpret_cast<uint4*>(&sA[buf][la[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) *reinterpret_cast<uint4*>(&sB[buf][lb[i]]) = rb[i];
  };

  v16f acc[2][2], tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = v16f{};
      tot[i][j] = v16f{};
    }

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) { sa[i] = nsa[i]; sb[i] = nsb[i]; }
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + l32;
        if constexpr (AF == 4) {
          const int c = s * 2 + half;
          const uint4 v = *reinterpret_cast<const uint4*>(&sA[buf][r * A_RB + ((c ^ swz<A_CH>(r)) * 16)]);
          af[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        } else {
          // E4M3 operand layout: dwords 0-3 hold K = 16*half + [0,16), dwords
          // 4-7 hold K = 32 + 16*half + [0,16) of this 64-wide K step
          const int c0 = s * 4 + half, c1 = s * 4 + 2 + half;
          const uint4 v0 = *reinterpret_cast<const uint4*>(&sA[buf][r * A_RB + ((c0 ^ swz<A_CH>(r)) * 16)]);
          const uint4 v1 = *reinterpret_cast<const uint4*>(&sA[buf][r * A_RB + ((c1 ^ swz<A_CH>(r)) * 16)]);
          af[i] = v8i{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                      (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        }
        const int rb2 = wn * 64 + i * 32 + l32;
        const int cb = s * 2 + half;
        const uint4 w = *reinterpret_cast<const uint4*>(&sB[buf][rb2 * B_RB + ((cb ^ swz<B_CH>(rb2)) * 16)]);
        bf[i] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (s == 0)
            acc[i][j] = mfma_scaled<0, AF>(af[i], bf[j], acc[i][j], (int)sa[i], (int)sb[j]);
          else
            acc[i][j] = mfma_scaled<2, AF>(af[i], bf[j], acc[i][j], (int)sa[i], (int)sb[j]);
        }
    }
    if constexpr (SLAB) {
      if ((kt + 1) % kSlabTiles == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            tot[i][j] += acc[i][j];
            acc[i][j] = v16f{};
          }
      }
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }
  if constexpr (SLAB) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] += tot[i][j];
  }
  epilogue<LR>(p, acc, 1.0f, m0, n0, wm, wn, lane);
}

template <int AF>
hipError_t dispatch(bool lr, bool slab, dim3 grid, const GemmP& p, hipStream_t s) {
  if (lr) {
    if (slab) gemm_mx_kernel<AF, true, true><<<grid, kThreads, 0, s>>>(p);
    else gemm_mx_kernel<AF, true, false><<<grid, kThreads, 0, s>>>(p);
  } else {
    if (slab) gemm_mx_kernel<AF, false, true><<<grid, kThreads, 0, s>>>(p);
    else gemm_mx_kernel<AF, false, false><<<grid, kThreads, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t s) {
  GemmP p;
  p.a = a.a_codes; p.lda = a.lda; p.as = a.a_scales; p.ldas = a.ld_as;
  p.w = a.w_codes; p.ldw = a.ldw; p.ws = a.w_scales; p.ldws = a.ld_ws;
  p.M = (int)a.M; p.N = (int)a.N; p.K = (int)a.K;
  p.tiles_m = (int)((a.M + BM - 1) / BM);
  p.tiles_n = (int)((a.N + BN - 1) / BN);
  p.col_map = a.col_map;
  p.u = a.u; p.ld_u = a.ld_u; p.l2t = a.l2t; p.rank = a.rank;
  p.bias = a.bias;
  p.out = a.out; p.ld_out = a.ld_out; p.n_out = (int)a.n_out;
  const dim3 grid(p.tiles_m * p.tiles_n);
  const bool lr = a.rank > 0;
  const bool slab = (a.K / BK) > 2 * kSlabTiles;
  return dispatch<4>(lr, slab, grid, p, s);
}

}  // namespace mxq
