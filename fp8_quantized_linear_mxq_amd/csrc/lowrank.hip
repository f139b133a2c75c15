// Low-rank down projection of the SVDQuant branch: u = x L1 (fp32 out).
//
// Nunchaku / SVDQuant article, "main explanation": a 16-bit low-rank part of
// each weight is kept next to the 4-bit residual; its first factor is applied
// to the unrotated, unquantized bf16 activations.  u stays fp32; the GEMM
// epilogue adds u L2.
//
// One workgroup covers 16 rows; its four waves split K four ways and each
// runs 16x16x32 bf16 MFMAs against L1^T ([rank][K], K contiguous, so both
// operands are 16-byte row loads), then the four partial tiles are summed in
// LDS.  Each wave's accumulation chain is K/128 MFMAs long.
#include "device_common.h"
#include "kernels.h"

namespace mxq {
namespace {

constexpr int kRows = 16;
constexpr int kMaxRank = 128;

__global__ __launch_bounds__(256) void lora_down_kernel(LoraDownArgs a) {
  __shared__ float part[4][kRows][kMaxRank];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * kRows;
  const int r16 = lane & 15, kq = lane >> 4;   // MFMA row / K-quarter of 8
  const int64_t row = m0 + r16 < a.rows ? m0 + r16 : a.rows - 1;
  const uint16_t* xr = a.x + row * a.ldx + kq * 8;
  const int nt = a.rank / 16;
  v4f acc[kMaxRank / 16];
#pragma unroll
  for (int t = 0; t < kMaxRank / 16; ++t) acc[t] = v4f{};
  const int ksteps = (int)(a.cols / 32);
  for (int ks = wave; ks < ksteps; ks += 4) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xr + ks * 32);
    const v8bf af = __builtin_bit_cast(v8bf, xv);
#pragma unroll
    for (int t = 0; t < kMaxRank / 16; ++t) {
      if (t < nt) {
        const uint4 lv = *reinterpret_cast<const uint4*>(a.l1t + (int64_t)(t * 16 + r16) * a.cols +
                                                         ks * 32 + kq * 8);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(v8bf, lv), acc[t],
                                                         0, 0, 0);
      }
    }
  }
  // 16x16 C layout: lane holds column lane%16, rows 4*(lane/16) + q
#pragma unroll
  for (int t = 0; t < kMaxRank / 16; ++t)
    if (t < nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) part[wave][4 * kq + q][t * 16 + r16] = acc[t][q];
  __syncthreads();
  for (int idx = tid; idx < kRows * a.rank; idx += 256) {
    const int r = idx / a.rank, c = idx % a.rank;
    if (m0 + r < a.rows)
      a.u[(m0 + r) * a.ld_u + c] = (part[0][r][c] + part[1][r][c]) + (part[2][r][c] + part[3][r][c]);
  }
}

}  // namespace

hipError_t launch_lora_down(const LoraDownArgs& a, hipStream_t s) {
  const int64_t blocks = (a.rows + kRows - 1) / kRows;
  if (blocks == 0) return hipSuccess;
  lora_down_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mxq
