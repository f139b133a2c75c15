// Block quantization kernels: MXFP4 / MXFP8 (E8M0 per 32), NVFP4 (E4M3 per 16
// + fp32 tensor scale, two passes when the tensor scale is dynamic) and INT4
// (fp32 per 32), each with an optional fused block-diagonal Hadamard rotation.
//
// Scale and rounding rules: "Bridging the Gap ... Microscaling FP4
// Quantization" summary, the two reasons FP4 fails (MXFP4 power-of-two
// scales, NVFP4 small groups with block and tensor scales); rotation: same
// page, modification 3 (block-diagonal Hadamard rotation of activations).
//
// Work layout: one lane per 32-element block of a row (cols is a multiple of
// 32): a lane loads 64 contiguous bytes of bf16 (128 of fp32), so a wave reads
// 4-8 KB of contiguous memory; the block amax (and the two NVFP4 16-block
// maxima) are in-lane; the 16/32-point Hadamard butterflies run in float64
// registers in-lane (128 points: two more stages across the block's 4 lanes);
// a lane's codes leave as one 16-byte (FP4/INT4) or 32-byte (FP8) store.
#include <atomic>

#include "device_common.h"
#include "grid_max.h"
#include "kernels.h"

namespace mxq {
namespace {

constexpr int kThreads = 256;

struct QParams {
  const void* x;
  int64_t ldx;
  uint32_t cpr;     // 8-element chunks per row
  uint32_t total;   // rows * cpr
  uint8_t* codes;
  int64_t ld_codes;
  uint8_t* scales;
  int64_t ld_scales;
  float* g_out;
  const float* g_static;
  const float* partials;
  int n_partials;
  unsigned* dbg;    // MXQ_DEBUG_CHECKS: set to 1 on a NaN / Inf input, else null
};

// One flag per device for the debug checks (NaN / Inf inputs); the host
// reads and clears it through its symbol address.
__device__ unsigned int g_nonfinite;

// Flags the device when any of a lane's loaded values is NaN or Inf (only
// with the debug checks on: dbg is null otherwise).
template <int N>
__device__ __forceinline__ void check_finite(const float* v, unsigned* dbg) {
  if (!dbg) return;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < N; ++i) bad |= !__builtin_isfinite(v[i]);
  if (bad) atomicOr(dbg, 1u);
}

template <int HAD>
__device__ constexpr double had_scale() {
  // float64 nearest to 1/sqrt(n): 1/4, sqrt(2)/8, sqrt(2)/16
  return HAD == 16 ? 0.25 : HAD == 32 ? 0x1.6a09e667f3bcdp-3 : 0x1.6a09e667f3bcdp-4;
}

template <int DT>
__device__ __forceinline__ void load_chunk(const QParams& p, uint32_t row, uint32_t col,
                                           bool active, float v[8]) {
  if constexpr (DT == DT_BF16) {
    uint4 q = make_uint4(0, 0, 0, 0);
    if (active)
      q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) +
                                          (int64_t)row * p.ldx + col);
    v[0] = bf16_bits_to_f32(q.x & 0xFFFFu); v[1] = bf16_bits_to_f32(q.x >> 16);
    v[2] = bf16_bits_to_f32(q.y & 0xFFFFu); v[3] = bf16_bits_to_f32(q.y >> 16);
    v[4] = bf16_bits_to_f32(q.z & 0xFFFFu); v[5] = bf16_bits_to_f32(q.z >> 16);
    v[6] = bf16_bits_to_f32(q.w & 0xFFFFu); v[7] = bf16_bits_to_f32(q.w >> 16);
  } else {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (active) {
      const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p.x) +
                                                        (int64_t)row * p.ldx + col);
      a = q[0];
      b = q[1];
    }
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ __forceinline__ float reduce_partials(const QParams& p) {
  // any workgroup of up to 1024 threads (whole waves)
  __shared__ float red[16];
  const int nw = (int)(blockDim.x >> 6);
  float m = 0.f;
  for (int i = threadIdx.x; i < p.n_partials; i += blockDim.x) m = fmaxf(m, p.partials[i]);
  m = group_max<64>(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w]);
  return m;
}

// Scale and element codes of one lane's 8 consecutive values of a block
// whose max |value| is amax (NVFP4: g is the tensor scale).  MX scales come
// from the exponent bits and the codes from the hardware scaled converts
// (exact RNE with saturation for a normal power-of-two scale) or threshold
// comparisons; NVFP4 / INT4 scales are correctly rounded float64 quotients.
template <int FMT>
__device__ __forceinline__ void encode8(const float v[8], float amax, float g, uint32_t code[8],
                                        uint32_t& sbyte, float& sfloat) {
  sbyte = 0;
  sfloat = 0.f;
  if constexpr (FMT == FMT_MXFP4) {
    const int e = mx_exponent(amax, 2);
    if (e >= -126) {
      // hardware RNE convert of x / 2**e, saturating at 6 (exact: the
      // scale is a normal power of two)
      const float sc = ldexpf(1.0f, e);
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const uint32_t b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[i], v[i + 1], sc, 0);
        code[i] = b & 0xFu;
        code[i + 1] = (b >> 4) & 0xFu;
      }
    } else {
      float th[7];
      e2m1_thresholds_pow2(e, th);
#pragma unroll
      for (int i = 0; i < 8; ++i) code[i] = e2m1_encode(v[i], th);
    }
    sbyte = (uint32_t)(e + 127);
  } else if constexpr (FMT == FMT_MXFP8) {
    const int e = mx_exponent(amax, 8);
    if (e >= -126) {
      // hardware RNE convert of x / 2**e; it does not saturate above 464,
      // so clamp to +-448 * 2**e first (every value there rounds to 448)
      const float sc = ldexpf(1.0f, e), lim = 448.0f * sc;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float x0 = fminf(fmaxf(v[i], -lim), lim);
        const float x1 = fminf(fmaxf(v[i + 1], -lim), lim);
        typedef short v2s __attribute__((ext_vector_type(2)));
        const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, x0, x1, sc, false);
        const uint32_t b = __builtin_bit_cast(uint32_t, r);
        code[i] = b & 0xFFu;
        code[i + 1] = (b >> 8) & 0xFFu;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) code[i] = e4m3_encode(ldexpf(v[i], -e));
    }
    sbyte = (uint32_t)(e + 127);
  } else if constexpr (FMT == FMT_NVFP4) {
    // s = RN_E4M3(amax / (6 g)) from the correctly rounded float64 quotient
    sbyte = (g == 0.f) ? 0u : e4m3_encode_f64((double)amax / (6.0 * (double)g));
    float th[7];
    e2m1_thresholds_sg(e4m3_value(sbyte), g, th);
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = e2m1_encode(v[i], th);
  } else {  // INT4: s = RN_fp32(amax / 7), q = clamp(RNE(x / s), -7, 7)
    sfloat = (float)((double)amax / 7.0);
    const double sd = (double)sfloat;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double q = (sfloat == 0.f) ? 0.0 : rint((double)v[i] / sd);
      q = fmin(7.0, fmax(-7.0, q));
      code[i] = (uint32_t)((int)q) & 0xFu;
    }
  }
}

// Store one lane's 8 codes (and, from the block's first lane, its scale).
template <int FMT>
__device__ __forceinline__ void store8(const QParams& p, uint32_t row, uint32_t col,
                                       const uint32_t code[8], uint32_t sbyte, float sfloat,
                                       bool scale_lane) {
  if constexpr (FMT == FMT_MXFP8) {
    uint2 w;
    w.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
    w.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
    *reinterpret_cast<uint2*>(p.codes + (int64_t)row * p.ld_codes + col) = w;
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= code[i] << (4 * i);
    *reinterpret_cast<uint32_t*>(p.codes + (int64_t)row * p.ld_codes + col / 2) = w;
  }
  if (scale_lane) {
    if constexpr (FMT == FMT_INT4) {
      *reinterpret_cast<float*>(p.scales + (int64_t)row * p.ld_scales + (col / 32) * 4) = sfloat;
    } else {
      const uint32_t blk = (FMT == FMT_NVFP4) ? col / 16 : col / 32;
      p.scales[(int64_t)row * p.ld_scales + blk] = (uint8_t)sbyte;
    }
  }
}

// NVFP4 tensor scale for this call (static, or g = RN_fp32(A / 2688) from the
// phase-1 partial maxima: the float64 quotient of two float32 values rounds
// correctly to float32, 53 >= 2*24 + 2); workgroup 0 publishes it.
template <int FMT>
__device__ __forceinline__ float tensor_scale(const QParams& p) {
  float g = 0.f;
  if constexpr (FMT == FMT_NVFP4) {
    g = p.g_static ? *p.g_static : (float)((double)reduce_partials(p) / 2688.0);
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.g_out) *p.g_out = g;
  }
  return g;
}

// Store one lane's whole 32-block: 32 codes (16 bytes FP4 / INT4, 32 bytes
// FP8) and its scales (one E8M0 byte, two E4M3 bytes for the NVFP4 16-blocks,
// or one fp32 INT4 scale).
template <int FMT>
__device__ __forceinline__ void store32(const QParams& p, int64_t row, int64_t col,
                                        const uint32_t (&code)[4][8], const uint32_t (&sbyte)[4],
                                        const float (&sfloat)[4]) {
  uint8_t* crow = p.codes + row * p.ld_codes;
  if constexpr (FMT == FMT_MXFP8) {
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[2 * j] = code[j][0] | (code[j][1] << 8) | (code[j][2] << 16) | (code[j][3] << 24);
      w[2 * j + 1] = code[j][4] | (code[j][5] << 8) | (code[j][6] << 16) | (code[j][7] << 24);
    }
    *reinterpret_cast<uint4*>(crow + col) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(crow + col + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w[j] |= code[j][i] << (4 * i);
    }
    *reinterpret_cast<uint4*>(crow + col / 2) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  uint8_t* srow = p.scales + row * p.ld_scales;
  if constexpr (FMT == FMT_INT4) {
    *reinterpret_cast<float*>(srow + (col / 32) * 4) = sfloat[0];
  } else if constexpr (FMT == FMT_NVFP4) {
    *reinterpret_cast<uint16_t*>(srow + col / 16) = (uint16_t)(sbyte[0] | (sbyte[2] << 8));
  } else {
    srow[col / 32] = (uint8_t)sbyte[0];
  }
}

// Scales and codes of one lane's 32-block held as v[4][8]: one amax for MX
// and INT4, one per 16 values for NVFP4.
template <int FMT>
__device__ __forceinline__ void encode32(const float (&v)[4][8], float g, uint32_t (&code)[4][8],
                                         uint32_t (&sbyte)[4], float (&sfloat)[4]) {
  float m[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m[j] = fmaxf(m[j], fabsf(v[j][i]));
  }
  float amax[4];
  if constexpr (FMT == FMT_NVFP4) {
    amax[0] = amax[1] = fmaxf(m[0], m[1]);
    amax[2] = amax[3] = fmaxf(m[2], m[3]);
  } else {
    amax[0] = amax[1] = amax[2] = amax[3] = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
  }
  if constexpr (FMT == FMT_NVFP4) {
    // one scale and one threshold set per 16-block (chunks 2h, 2h + 1)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t sb = (g == 0.f) ? 0u : e4m3_encode_f64((double)amax[2 * h] / (6.0 * (double)g));
      float th[7];
      e2m1_thresholds_sg(e4m3_value(sb), g, th);
#pragma unroll
      for (int j = 2 * h; j < 2 * h + 2; ++j) {
        sbyte[j] = sb;
        sfloat[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) code[j][i] = e2m1_encode(v[j][i], th);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) encode8<FMT>(v[j], amax[j], g, code[j], sbyte[j], sfloat[j]);
  }
}

// A lane's 32 consecutive values of one row (64 contiguous bytes of bf16,
// 128 of fp32).
template <int DT>
__device__ __forceinline__ void load32(const QParams& p, int64_t row, int64_t col, float (&v)[4][8]) {
  if constexpr (DT == DT_BF16) {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + row * p.ldx + col);
    uint4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = q[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t d[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[j][2 * i] = bf16_bits_to_f32(d[i] & 0xFFFFu);
        v[j][2 * i + 1] = bf16_bits_to_f32(d[i] >> 16);
      }
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p.x) + row * p.ldx + col);
    float4 w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = q[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j][0] = w[2 * j].x; v[j][1] = w[2 * j].y; v[j][2] = w[2 * j].z; v[j][3] = w[2 * j].w;
      v[j][4] = w[2 * j + 1].x; v[j][5] = w[2 * j + 1].y; v[j][6] = w[2 * j + 1].z; v[j][7] = w[2 * j + 1].w;
    }
  }
}

// Block-diagonal Hadamard of a lane's 32 values (element index 8j + i):
// butterfly stages at distances 1 .. min(n, 32) / 2 in registers, then for
// n = 128 across the 4 lanes that hold the block (lane distance 1, 2 =
// element distance 32, 64); sums exact in float64, r = RN_fp32(RN_fp64(c_n S)).
template <int HAD>
__device__ __forceinline__ void hadamard32(float (&v)[4][8], int lane) {
  double h[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) h[e] = (double)v[e >> 3][e & 7];
  constexpr int IN = HAD < 32 ? HAD : 32;
#pragma unroll
  for (int d = 1; d < IN; d <<= 1) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if (e & d) continue;
      const double a = h[e], b = h[e + d];
      h[e] = a + b;
      h[e + d] = a - b;
    }
  }
  if constexpr (HAD == 128) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bool upper = (lane & (1 << st)) != 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const double o = st == 0 ? xor_lane_d<1>(h[e]) : xor_lane_d<2>(h[e]);
        h[e] = upper ? (o - h[e]) : (h[e] + o);
      }
    }
  }
  constexpr double c = had_scale<HAD>();
  // an exactly-zero sum is the real zero: + 0.0 turns -0 into +0
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e >> 3][e & 7] = (float)(c * (h[e] + 0.0));
}

// Quantize with one lane per 32-block (32 consecutive values of a row):
// coalesced 64-byte (bf16) runs per lane, in-lane amax and rotation
// (16 / 32 points; 128 points across 4 lanes), one 16/32-byte code store per
// lane.  Grid-stride over the rows * cols / 32 blocks.
template <int DT, int FMT, int HAD>
__global__ __launch_bounds__(kThreads) void quantize32_kernel(QParams p, uint32_t bpr, uint32_t nblk) {
  const float g = tensor_scale<FMT>(p);
  const int lane = threadIdx.x & 63;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b - lane < nblk; b += stride) {
    // whole waves stay in the loop (the 128-point rotation exchanges lanes);
    // lanes past the end work on a clamped block and store nothing
    const bool act = b < nblk;
    const uint32_t bb = act ? b : nblk - 1;
    const int64_t row = bb / bpr, col = (int64_t)(bb - (uint32_t)row * bpr) * 32;
    float v[4][8];
    load32<DT>(p, row, col, v);
    check_finite<32>(&v[0][0], p.dbg);
    if constexpr (HAD > 0) hadamard32<HAD>(v, lane);
    uint32_t code[4][8], sbyte[4];
    float sfloat[4];
    encode32<FMT>(v, g, code, sbyte, sfloat);
    if (act) store32<FMT>(p, row, col, code, sbyte, sfloat);
  }
}

// NVFP4 phase 1 in the same layout: per-workgroup max |r|.
template <int DT, int HAD>
__global__ __launch_bounds__(kThreads) void amax32_kernel(QParams p, float* partials, uint32_t bpr,
                                                          uint32_t nblk) {
  const int lane = threadIdx.x & 63;
  const uint32_t stride = gridDim.x * kThreads;
  float m = 0.f;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b - lane < nblk; b += stride) {
    const bool act = b < nblk;
    const uint32_t bb = act ? b : nblk - 1;
    const int64_t row = bb / bpr, col = (int64_t)(bb - (uint32_t)row * bpr) * 32;
    float v[4][8];
    load32<DT>(p, row, col, v);
    check_finite<32>(&v[0][0], p.dbg);
    if constexpr (HAD > 0) hadamard32<HAD>(v, lane);
    if (act) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
    }
  }
  __shared__ float red[kThreads / 64];
  m = group_max<64>(m);
  if (lane == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
    partials[blockIdx.x] = r;
  }
}

// One-pass NVFP4 with the dynamic tensor scale.  The tensor scale depends on
// the amax of the whole (rotated) tensor, which the two-pass form gets by
// reading x twice.  Here every lane keeps its J rotated 32-blocks in
// registers; the workgroups' maxima meet in a device-wide maximum
// (grid_max.h) that every workgroup waits for, and the blocks are encoded
// from the registers, so x is read once.  The wait needs every workgroup
// resident at once: the host sizes the grid from the kernel's occupancy on
// this device (the two-pass kernels take inputs that do not fit).  A call
// whose grid could not become resident within about a second (other work
// holding the compute units) writes a NaN tensor scale.  Consecutive calls
// take different barrier slots of a small ring (a static array per device,
// zero at load; kernels get its device address, looked up once per device);
// calls ordered on one stream reuse them safely.
constexpr int kNvSlots = 16;
static __device__ __align__(256) GridMaxSlot g_nvslot[kNvSlots];

template <int DT, int HAD, int J>
__global__ __launch_bounds__(kThreads) void nvfp4_onepass_kernel(QParams p, uint32_t bpr,
                                                                 uint32_t nblk, GridMaxSlot* slot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t b0 = blockIdx.x * (kThreads * J) + threadIdx.x;
  float v[J][4][8];
  uint32_t rows[J], cols[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    // lanes past the end work on a clamped block (the 128-point rotation
    // exchanges lanes) and neither count nor store it
    const uint32_t b = b0 + j * kThreads;
    const uint32_t bb = b < nblk ? b : nblk - 1;
    rows[j] = bb / bpr;
    cols[j] = (bb - rows[j] * bpr) * 32;
    load32<DT>(p, rows[j], cols[j], v[j]);
  }
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    check_finite<32>(&v[j][0][0], p.dbg);
    if constexpr (HAD > 0) hadamard32<HAD>(v[j], lane);
    if (b0 + j * kThreads < nblk) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][k][i]));
    }
  }
  __shared__ float red[kThreads / 64];
  __shared__ float g_sh;
  m = group_max<64>(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (wave == 0) {
    float wm = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) wm = fmaxf(wm, red[w]);
    const float A = grid_max_wave0(slot, wm);
    // g = RN_fp32(A / 2688): the float64 quotient of two float32 values
    // rounds correctly to float32 (a NaN from a timed-out wait passes on)
    const float g = (float)((double)A / 2688.0);
    if (lane == 0) {
      g_sh = g;
      if (blockIdx.x == 0 && p.g_out) *p.g_out = g;
    }
  }
  __syncthreads();
  const float g = g_sh;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (b0 + j * kThreads >= nblk) continue;
    uint32_t code[4][8], sbyte[4];
    float sfloat[4];
    encode32<FMT_NVFP4>(v[j], g, code, sbyte, sfloat);
    store32<FMT_NVFP4>(p, rows[j], cols[j], code, sbyte, sfloat);
  }
}

// Quantize fused with the low-rank down projection u = x L1 of the SVDQuant
// branch (Nunchaku article, "main explanation": the 16-bit low-rank part
// reads the same unrotated activations).  One workgroup owns 16 rows; its
// eight waves take every eighth 128-column group.  Lane (r, q) = (lane % 16,
// lane / 16) loads the 64 contiguous bytes of row r, columns 32q + [0, 32)
// of the group -- exactly one 32-block (two NVFP4 16-blocks), so the block
// amax needs no lane exchange and its codes leave as one 16-byte (FP4) or
// 32-byte (FP8) store -- and the same registers are the four K-steps of
// 16x16x32 bf16 MFMAs against L1^T: step j pairs x columns 32q + 8j + [0, 8)
// with the same columns of L1^T, a consistent reordering of the sum.  The
// waves' partial u tiles are summed in LDS.  bf16 input, no rotation,
// columns a multiple of 128.
constexpr int kLrRows = 16;
constexpr int kLrWaves = 8;

template <int FMT, int NT, bool PK>
__global__ __launch_bounds__(64 * kLrWaves) void quantize_lr_kernel(QParams p, LoraDownArgs lr) {
  __shared__ float part[kLrWaves][kLrRows][16 * NT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float g = tensor_scale<FMT>(p);
  const int64_t m0 = (int64_t)blockIdx.x * kLrRows;
  const int r16 = lane & 15, kq = lane >> 4;
  const bool row_ok = m0 + r16 < lr.rows;
  const int64_t row = row_ok ? m0 + r16 : lr.rows - 1;
  const uint16_t* xr = lr.x + row * lr.ldx + kq * 32;
  // L1^T fragments: [rank][cols] rows (a lane's 16 bytes of one rank row,
  // 64 bytes apart across the lane's K-quarter: 32 cache lines per wave load)
  // or the packed order (one contiguous kilobyte per wave load; the
  // fragment reads of the kernel cost about a quarter less time).
  const uint16_t* lp = PK ? lr.l1t + lane * 8 : lr.l1t + (int64_t)r16 * lr.cols + kq * 32;
  const int groups = (int)(lr.cols / 128);
  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{};
  // one group in flight per wave: loading the next group's operands ahead
  // (two in flight) measured 6% slower on 4096 x 3072 at rank 32
  for (int gi = wave; gi < groups; gi += kLrWaves) {
    uint4 xv[4], lv[NT][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[j] = *reinterpret_cast<const uint4*>(xr + gi * 128 + 8 * j);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        lv[t][j] = *reinterpret_cast<const uint4*>(PK ? lp + (((int64_t)gi * NT + t) * 4 + j) * 512
                                                      : lp + (int64_t)t * 16 * lr.cols + gi * 128 + 8 * j);
    }
    {
      float v[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[j][2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
          v[j][2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
        }
      }
      check_finite<32>(&v[0][0], p.dbg);
      float m[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m[j] = fmaxf(m[j], fabsf(v[j][i]));
      }
      float amax[4];
      if constexpr (FMT == FMT_NVFP4) {
        amax[0] = amax[1] = fmaxf(m[0], m[1]);
        amax[2] = amax[3] = fmaxf(m[2], m[3]);
      } else {
        amax[0] = amax[1] = amax[2] = amax[3] = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
      }
      uint32_t code[4][8], sbyte[4];
      float sfloat[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) encode8<FMT>(v[j], amax[j], g, code[j], sbyte[j], sfloat[j]);
      if (row_ok) {
        const int64_t col = (int64_t)gi * 128 + kq * 32;
        uint8_t* crow = p.codes + row * p.ld_codes;
        if constexpr (FMT == FMT_MXFP8) {
          uint32_t w[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            w[2 * j] = code[j][0] | (code[j][1] << 8) | (code[j][2] << 16) | (code[j][3] << 24);
            w[2 * j + 1] = code[j][4] | (code[j][5] << 8) | (code[j][6] << 16) | (code[j][7] << 24);
          }
          *reinterpret_cast<uint4*>(crow + col) = make_uint4(w[0], w[1], w[2], w[3]);
          *reinterpret_cast<uint4*>(crow + col + 16) = make_uint4(w[4], w[5], w[6], w[7]);
        } else {
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            w[j] = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) w[j] |= code[j][i] << (4 * i);
          }
          *reinterpret_cast<uint4*>(crow + col / 2) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        uint8_t* srow = p.scales + row * p.ld_scales;
        if constexpr (FMT == FMT_INT4) {
          *reinterpret_cast<float*>(srow + (col / 32) * 4) = sfloat[0];
        } else if constexpr (FMT == FMT_NVFP4) {
          *reinterpret_cast<uint16_t*>(srow + col / 16) = (uint16_t)(sbyte[0] | (sbyte[2] << 8));
        } else {
          srow[col / 32] = (uint8_t)sbyte[0];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8bf af = __builtin_bit_cast(v8bf, xv[j]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(v8bf, lv[t][j]),
                                                           acc[t], 0, 0, 0);
      }
    }
  }
  // 16x16 C layout: lane holds column lane % 16, rows 4 * (lane / 16) + q
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) part[wave][4 * kq + q][t * 16 + r16] = acc[t][q];
  __syncthreads();
  for (int idx = tid; idx < kLrRows * 16 * NT; idx += 64 * kLrWaves) {
    const int r = idx / (16 * NT), c = idx % (16 * NT);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kLrWaves; ++w) sum += part[w][r][c];
    if (m0 + r < lr.rows) lr.u[(m0 + r) * lr.ld_u + c] = sum;
  }
}

template <int FMT, bool PK>
hipError_t launch_lr_pk(int nt, dim3 grid, const QParams& p, const LoraDownArgs& lr, hipStream_t s) {
  switch (nt) {
    case 1: quantize_lr_kernel<FMT, 1, PK><<<grid, 64 * kLrWaves, 0, s>>>(p, lr); break;
    case 2: quantize_lr_kernel<FMT, 2, PK><<<grid, 64 * kLrWaves, 0, s>>>(p, lr); break;
    case 3: quantize_lr_kernel<FMT, 3, PK><<<grid, 64 * kLrWaves, 0, s>>>(p, lr); break;
    case 4: quantize_lr_kernel<FMT, 4, PK><<<grid, 64 * kLrWaves, 0, s>>>(p, lr); break;
    case 5: quantize_lr_kernel<FMT, 5, PK><<<grid, 64 * kLrWaves, 0, s>>>(p, lr); break;
    case 6: quantize_lr_kernel<FMT, 6, PK><<<grid, 64 * kLrWaves, 0, s>>>(p, lr); break;
    case 7: quantize_lr_kernel<FMT, 7, PK><<<grid, 64 * kLrWaves, 0, s>>>(p, lr); break;
    case 8: quantize_lr_kernel<FMT, 8, PK><<<grid, 64 * kLrWaves, 0, s>>>(p, lr); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_lr(int nt, dim3 grid, const QParams& p, const LoraDownArgs& lr, hipStream_t s) {
  return lr.packed ? launch_lr_pk<FMT, true>(nt, grid, p, lr, s)
                   : launch_lr_pk<FMT, false>(nt, grid, p, lr, s);
}

// One thread per 16-byte piece of the packed order (see launch_pack_l1t).
__global__ __launch_bounds__(256) void pack_l1t_kernel(const uint16_t* l1t, int nt, int64_t cols,
                                                       uint16_t* l1p, int64_t pieces) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int lane = (int)(i & 63), j = (int)((i >> 6) & 3);
  const int64_t rest = i >> 8;
  const int t = (int)(rest % nt);
  const int64_t g = rest / nt;
  const uint16_t* src = l1t + (int64_t)(t * 16 + (lane & 15)) * cols + g * 128 + (lane >> 4) * 32 + 8 * j;
  *reinterpret_cast<uint4*>(l1p + i * 8) = *reinterpret_cast<const uint4*>(src);
}

// ---------------------------------------------------------------------------
// Per-output-channel format selection (Chameleon article, "the format is
// chosen by the value distribution": try the available formats per output
// channel, keep the least reconstruction error).  One workgroup per weight
// row; every candidate's codes come from the same encoders as the quantize
// kernel, and each squared error is exact in float64.
// ---------------------------------------------------------------------------

__device__ __forceinline__ double e2m1_mag(uint32_t c) {
  const uint32_t m = c & 7u, e = m >> 1, man = m & 1u;
  const double v = (e == 0) ? 0.5 * (double)man : ldexp(1.0 + 0.5 * (double)man, (int)e - 1);
  return (c & 8u) ? -v : v;
}

struct SelParams {
  QParams q;            // x = w, cpr, total (per row: cpr chunks)
  int n_cand;
  int cand[4];
  double* sse;          // [n][n_cand]
  uint8_t* choice;      // [n]
};

template <int DT>
__global__ __launch_bounds__(kThreads) void select_kernel(SelParams sp) {
  const QParams& p = sp.q;
  const int lane = threadIdx.x & 63;
  float g = (float)((double)reduce_partials(p) / 2688.0);
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.g_out) *p.g_out = g;
  const uint32_t row = blockIdx.x;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (uint32_t base = 0; base < p.cpr; base += kThreads) {
    const uint32_t c = base + threadIdx.x;
    const bool act = c < p.cpr;
    float v[8];
    load_chunk<DT>(p, row, act ? c * 8u : 0u, act, v);
    check_finite<8>(v, p.dbg);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    const float a32 = group_max<4>(m), a16 = group_max<2>(m);
    for (int ci = 0; ci < sp.n_cand; ++ci) {
      double e2 = 0.0;
      const int f = sp.cand[ci];
      if (f == FMT_MXFP4) {
        const int e = mx_exponent(a32, 2);
        float th[7];
        e2m1_thresholds_pow2(e, th);
        const double sc = ldexp(1.0, e);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double d = (double)v[i] - e2m1_mag(e2m1_encode(v[i], th)) * sc;
          e2 += d * d;
        }
      } else if (f == FMT_NVFP4) {
        const uint32_t sb = (g == 0.f) ? 0u : e4m3_encode_f64((double)a16 / (6.0 * (double)g));
        const double dsc = (double)e4m3_value(sb) * (double)g;
        float th[7];
        e2m1_thresholds_f64(dsc, th);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double d = (double)v[i] - e2m1_mag(e2m1_encode(v[i], th)) * dsc;
          e2 += d * d;
        }
      } else {  // INT4
        const float s = (float)((double)a32 / 7.0);
        const double sd = (double)s;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          double q = (s == 0.f) ? 0.0 : rint((double)v[i] / sd);
          q = fmin(7.0, fmax(-7.0, q));
          const double d = (double)v[i] - q * sd;
          e2 += d * d;
        }
      }
      acc[ci] += act ? e2 : 0.0;
    }
  }
  __shared__ double red[4][kThreads / 64];
  for (int ci = 0; ci < sp.n_cand; ++ci) {
    double t = acc[ci];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
    if (lane == 0) red[ci][threadIdx.x >> 6] = t;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int best = 0;
    double best_v = 0.0;
    for (int ci = 0; ci < sp.n_cand; ++ci) {
      const double t = (red[ci][0] + red[ci][1]) + (red[ci][2] + red[ci][3]);
      sp.sse[(int64_t)row * sp.n_cand + ci] = t;
      if (ci == 0 || t < best_v) { best = ci; best_v = t; }
    }
    sp.choice[row] = (uint8_t)best;
  }
}

// Stable grouping of rows by chosen candidate: counts and permutation.
__global__ __launch_bounds__(256) void group_kernel(const uint8_t* choice, int n, int n_cand,
                                                    int32_t* perm, int32_t* counts) {
  __shared__ int cnt[256][4];
  __shared__ int base[4];
  const int t = threadIdx.x;
  const int per = (n + 255) / 256;
  const int lo = t * per, hi = min(n, lo + per);
  int c[4] = {0, 0, 0, 0};
  for (int r = lo; r < hi; ++r) c[choice[r]]++;
  for (int k = 0; k < 4; ++k) cnt[t][k] = c[k];
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int k = 0; k < n_cand; ++k) {
      base[k] = run;
      int s = 0;
      for (int i = 0; i < 256; ++i) { const int v = cnt[i][k]; cnt[i][k] = s; s += v; }
      if (counts) counts[k] = s;
      run += s;
    }
  }
  __syncthreads();
  if (perm) {
    int pos[4];
    for (int k = 0; k < 4; ++k) pos[k] = (k < n_cand) ? base[k] + cnt[t][k] : 0;
    for (int r = lo; r < hi; ++r) perm[pos[choice[r]]++] = r;
  }
}

// g = RN_fp32(A / 2688) from the phase-1 partial maxima, written to g_out
// (one workgroup).
__global__ __launch_bounds__(kThreads) void tensor_scale_kernel(QParams p) {
  const float g = (float)((double)reduce_partials(p) / 2688.0);
  if (threadIdx.x == 0) *p.g_out = g;
}

template <int DT, int FMT>
hipError_t dispatch_had(int had, dim3 grid, const QParams& p, uint32_t bpr, uint32_t nblk,
                        hipStream_t s) {
  switch (had) {
    case 0: quantize32_kernel<DT, FMT, 0><<<grid, kThreads, 0, s>>>(p, bpr, nblk); break;
    case 16: quantize32_kernel<DT, FMT, 16><<<grid, kThreads, 0, s>>>(p, bpr, nblk); break;
    case 32: quantize32_kernel<DT, FMT, 32><<<grid, kThreads, 0, s>>>(p, bpr, nblk); break;
    case 128: quantize32_kernel<DT, FMT, 128><<<grid, kThreads, 0, s>>>(p, bpr, nblk); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t dispatch_fmt(int fmt, int had, dim3 grid, const QParams& p, uint32_t bpr, uint32_t nblk,
                        hipStream_t s) {
  switch (fmt) {
    case FMT_MXFP4: return dispatch_had<DT, FMT_MXFP4>(had, grid, p, bpr, nblk, s);
    case FMT_MXFP8: return dispatch_had<DT, FMT_MXFP8>(had, grid, p, bpr, nblk, s);
    case FMT_NVFP4: return dispatch_had<DT, FMT_NVFP4>(had, grid, p, bpr, nblk, s);
    case FMT_INT4: return dispatch_had<DT, FMT_INT4>(had, grid, p, bpr, nblk, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t dispatch_amax(int had, dim3 grid, const QParams& p, float* partials, uint32_t bpr,
                         uint32_t nblk, hipStream_t s) {
  switch (had) {
    case 0: amax32_kernel<DT, 0><<<grid, kThreads, 0, s>>>(p, partials, bpr, nblk); break;
    case 16: amax32_kernel<DT, 16><<<grid, kThreads, 0, s>>>(p, partials, bpr, nblk); break;
    case 32: amax32_kernel<DT, 32><<<grid, kThreads, 0, s>>>(p, partials, bpr, nblk); break;
    case 128: amax32_kernel<DT, 128><<<grid, kThreads, 0, s>>>(p, partials, bpr, nblk); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Workgroups of nvfp4_onepass_kernel<DT, HAD, J> the current device holds
// at once (occupancy x compute units), looked up once per device; 0 when
// unknown (the caller then takes the two-pass kernels).
template <int DT, int HAD, int J>
int onepass_capacity() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int c = cache[dev].load(std::memory_order_acquire);
  if (c == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, nvfp4_onepass_kernel<DT, HAD, J>,
                                                     kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    c = per_cu > 0 && cus > 0 ? per_cu * cus : -1;
    cache[dev].store(c, std::memory_order_release);
  }
  return c > 0 ? c : 0;
}

std::atomic<unsigned> g_next_nvslot{0};

// Device address of the current device's barrier-slot ring (its own copy
// of g_nvslot), looked up with that device current, once per device.
GridMaxSlot* nvslot_ring() {
  constexpr int kMaxDev = 64;
  static std::atomic<GridMaxSlot*> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  GridMaxSlot* ptr = cache[dev].load(std::memory_order_acquire);
  if (!ptr) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(g_nvslot)) != hipSuccess || !a) return nullptr;
    ptr = static_cast<GridMaxSlot*>(a);
    cache[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

// The one-pass kernel with J blocks per lane, if its grid is resident at
// once on this device; false leaves the work to the two-pass kernels.
template <int DT, int HAD, int J>
bool onepass_j(const QParams& p, uint32_t bpr, uint32_t nblk, hipStream_t s, hipError_t* err) {
  const uint64_t grid = ((uint64_t)nblk + kThreads * J - 1) / (kThreads * J);
  if (grid > (uint64_t)onepass_capacity<DT, HAD, J>() || grid > (uint64_t)kGridMaxWgs) return false;
  GridMaxSlot* ring = nvslot_ring();
  if (!ring) return false;
  const int slot = (int)(g_next_nvslot.fetch_add(1u, std::memory_order_relaxed) % kNvSlots);
  nvfp4_onepass_kernel<DT, HAD, J><<<dim3((unsigned)grid), kThreads, 0, s>>>(p, bpr, nblk,
                                                                             ring + slot);
  *err = hipGetLastError();
  return true;
}

// The fewest blocks per lane (the most workgroups) that fit.
template <int DT, int HAD>
bool onepass_had(const QParams& p, uint32_t bpr, uint32_t nblk, hipStream_t s, hipError_t* err) {
  return onepass_j<DT, HAD, 1>(p, bpr, nblk, s, err) || onepass_j<DT, HAD, 2>(p, bpr, nblk, s, err) ||
         onepass_j<DT, HAD, 4>(p, bpr, nblk, s, err);
}

template <int DT>
bool onepass(int had, const QParams& p, uint32_t bpr, uint32_t nblk, hipStream_t s,
             hipError_t* err) {
  switch (had) {
    case 0: return onepass_had<DT, 0>(p, bpr, nblk, s, err);
    case 16: return onepass_had<DT, 16>(p, bpr, nblk, s, err);
    case 32: return onepass_had<DT, 32>(p, bpr, nblk, s, err);
    case 128: return onepass_had<DT, 128>(p, bpr, nblk, s, err);
    default: return false;
  }
}

}  // namespace

// Scratch of the allocation-free quantize entry point: room for the NVFP4
// tensor-amax partials (one float per amax workgroup, at most kAmaxPartials)
// on each device, held until the process ends.  Only its device address,
// looked up once per device, is ever passed to a kernel.
static __device__ __align__(256) float scratch[kAmaxPartials];

hipError_t quantize_scratch(void** out, size_t* bytes) {
  constexpr int kMaxDev = 64;
  static std::atomic<void*> cache[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  void* ptr = cache[dev].load(std::memory_order_acquire);
  if (!ptr) {
    // with this device current: its own copy of the array
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    cache[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  *bytes = sizeof(scratch);
  return hipSuccess;
}

hipError_t nonfinite_flag_ptr(unsigned** out) {
  // the flag's address on the current device, looked up once per device
  constexpr int kMaxDev = 64;
  static std::atomic<unsigned*> cache[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  unsigned* flag = cache[dev].load(std::memory_order_acquire);
  if (!flag) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_nonfinite));
    if (e != hipSuccess) return e;
    flag = static_cast<unsigned*>(ptr);
    cache[dev].store(flag, std::memory_order_release);
  }
  *out = flag;
  return hipSuccess;
}

hipError_t launch_pack_l1t(const uint16_t* l1t, int rank, int64_t cols, uint16_t* l1p,
                           hipStream_t s) {
  const int64_t pieces = (int64_t)rank * cols / 8;
  if (pieces == 0) return hipSuccess;
  pack_l1t_kernel<<<dim3((unsigned)((pieces + 255) / 256)), 256, 0, s>>>(l1t, rank / 16, cols, l1p,
                                                                        pieces);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t s) {
  QParams p;
  p.x = a.x;
  p.ldx = a.ldx;
  p.cpr = (uint32_t)(a.cols / 8);
  p.total = (uint32_t)(a.rows * (a.cols / 8));
  p.codes = a.codes;
  p.ld_codes = a.ld_codes;
  p.scales = a.scales;
  p.ld_scales = a.ld_scales;
  p.g_out = a.tensor_scale_out;
  p.g_static = a.static_tensor_scale;
  p.partials = a.partials;
  p.n_partials = 0;
  p.dbg = a.dbg;

  // one lane per 32-block
  const uint32_t bpr = (uint32_t)(a.cols / 32);
  const uint32_t nblk = (uint32_t)(a.rows * bpr);
  uint32_t blocks = (nblk + kThreads - 1) / kThreads;
  if (blocks > 8192u) blocks = 8192u;
  if (blocks == 0) return hipSuccess;

  if (a.fmt == FMT_NVFP4 && a.static_tensor_scale == nullptr) {
    // one pass over x when the blocks fit in the registers of one resident grid
    if (!(a.lr && a.lr->rank > 0) && !a.nv_two_pass) {
      hipError_t e = hipSuccess;
      const bool done = (a.dtype == DT_BF16) ? onepass<DT_BF16>(a.hadamard_n, p, bpr, nblk, s, &e)
                                             : onepass<DT_F32>(a.hadamard_n, p, bpr, nblk, s, &e);
      if (done) return e;
    }
    uint32_t pb = blocks < (uint32_t)kAmaxPartials ? blocks : (uint32_t)kAmaxPartials;
    p.n_partials = (int)pb;
    hipError_t e = (a.dtype == DT_BF16)
                       ? dispatch_amax<DT_BF16>(a.hadamard_n, dim3(pb), p, a.partials, bpr, nblk, s)
                       : dispatch_amax<DT_F32>(a.hadamard_n, dim3(pb), p, a.partials, bpr, nblk, s);
    if (e != hipSuccess) return e;
  }
  if (a.lr && a.lr->rank > 0) {
    if (a.dtype == DT_BF16 && a.hadamard_n == 0 && a.lr->rank <= 128 && a.cols % 128 == 0) {
      const dim3 g((unsigned)((a.rows + kLrRows - 1) / kLrRows));
      const int nt = a.lr->rank / 16;
      switch (a.fmt) {
        case FMT_MXFP4: return launch_lr<FMT_MXFP4>(nt, g, p, *a.lr, s);
        case FMT_MXFP8: return launch_lr<FMT_MXFP8>(nt, g, p, *a.lr, s);
        case FMT_NVFP4: return launch_lr<FMT_NVFP4>(nt, g, p, *a.lr, s);
        case FMT_INT4: return launch_lr<FMT_INT4>(nt, g, p, *a.lr, s);
        default: return hipErrorInvalidValue;
      }
    }
    // the packed order is read by the fused kernel only (its conditions are
    // checked before any launch)
    if (a.lr->packed) return hipErrorInvalidValue;
    // rotated activations (or columns not a multiple of 128): quantize, then
    // u from the unrotated x in its own pass
    hipError_t e = (a.dtype == DT_BF16)
                       ? dispatch_fmt<DT_BF16>(a.fmt, a.hadamard_n, dim3(blocks), p, bpr, nblk, s)
                       : dispatch_fmt<DT_F32>(a.fmt, a.hadamard_n, dim3(blocks), p, bpr, nblk, s);
    if (e != hipSuccess) return e;
    return launch_lora_down(*a.lr, s);
  }
  return (a.dtype == DT_BF16)
             ? dispatch_fmt<DT_BF16>(a.fmt, a.hadamard_n, dim3(blocks), p, bpr, nblk, s)
             : dispatch_fmt<DT_F32>(a.fmt, a.hadamard_n, dim3(blocks), p, bpr, nblk, s);
}


hipError_t launch_nvfp4_tensor_scale(const void* x, int dtype, int64_t rows, int64_t cols,
                                     int64_t ldx, float* partials, float* g_out,
                                     unsigned* dbg, hipStream_t s) {
  QParams p;
  p.x = x;
  p.ldx = ldx;
  p.cpr = (uint32_t)(cols / 8);
  p.total = (uint32_t)(rows * (cols / 8));
  p.codes = nullptr; p.ld_codes = 0; p.scales = nullptr; p.ld_scales = 0;
  p.g_out = g_out;
  p.g_static = nullptr;
  p.partials = partials;
  p.dbg = dbg;
  const uint32_t bpr = (uint32_t)(cols / 32), nblk = (uint32_t)(rows * bpr);
  uint32_t blocks = (nblk + kThreads - 1) / kThreads;
  if (blocks > (uint32_t)kAmaxPartials) blocks = kAmaxPartials;
  if (blocks == 0) return hipSuccess;
  p.n_partials = (int)blocks;
  hipError_t e = (dtype == DT_BF16)
                     ? dispatch_amax<DT_BF16>(0, dim3(blocks), p, partials, bpr, nblk, s)
                     : dispatch_amax<DT_F32>(0, dim3(blocks), p, partials, bpr, nblk, s);
  if (e != hipSuccess) return e;
  tensor_scale_kernel<<<1, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  SelParams sp;
  QParams& p = sp.q;
  p.x = a.w;
  p.ldx = a.ldw;
  p.cpr = (uint32_t)(a.k / 8);
  p.total = (uint32_t)(a.n * (a.k / 8));
  p.codes = nullptr; p.ld_codes = 0; p.scales = nullptr; p.ld_scales = 0;
  p.g_out = a.g_out ? a.g_out : a.g_ws;
  p.g_static = nullptr;
  p.partials = a.partials;
  p.dbg = a.dbg;
  if (a.n == 0) return hipSuccess;
  const uint32_t bpr = (uint32_t)(a.k / 32), nblk = (uint32_t)(a.n * bpr);
  uint32_t blocks = (nblk + kThreads - 1) / kThreads;
  if (blocks > (uint32_t)kAmaxPartials) blocks = kAmaxPartials;
  p.n_partials = (int)blocks;
  hipError_t e = (a.dtype == DT_BF16)
                     ? dispatch_amax<DT_BF16>(0, dim3(blocks), p, a.partials, bpr, nblk, s)
                     : dispatch_amax<DT_F32>(0, dim3(blocks), p, a.partials, bpr, nblk, s);
  if (e != hipSuccess) return e;
  sp.n_cand = a.n_cand;
  for (int i = 0; i < 4; ++i) sp.cand[i] = i < a.n_cand ? a.cand[i] : 0;
  sp.sse = a.sse ? a.sse : a.sse_ws;
  sp.choice = a.choice;
  if (a.dtype == DT_BF16) select_kernel<DT_BF16><<<dim3((unsigned)a.n), kThreads, 0, s>>>(sp);
  else select_kernel<DT_F32><<<dim3((unsigned)a.n), kThreads, 0, s>>>(sp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.perm || a.counts) {
    group_kernel<<<1, 256, 0, s>>>(a.choice, (int)a.n, a.n_cand, a.perm, a.counts);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace mxq
