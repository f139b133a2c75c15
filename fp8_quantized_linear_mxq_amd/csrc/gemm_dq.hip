// GEMM route for INT4 weight rows (Chameleon palette: symmetric int4 with an
// fp32 scale per 32), against MXFP8, NVFP4 or MXFP4 activations, or
// unquantized bf16 activations (4-bit weights, 16-bit activations).
//
// The arbitrary fp32 weight scale cannot fold into a 16-bit operand, so each
// 32-element block's partial sum comes from two bf16 MFMAs on the integer
// codes (exact in bf16) and is scaled into an fp32 accumulator with one FMA
// per output element.  Activations are dequantized exactly to 16-bit (see
// gemm_dqp.hip for why the E4M3 MFMAs are not used): E4M3 x E8M0 and
// E2M1 x E8M0 have <= 4 significant bits, E2M1 x E4M3 (NVFP4) <= 6 bits;
// NVFP4 tensor scales are applied in the epilogue.
//
// Tile 128x128, K-tile 64, 2x2 waves of 64x64, 32x32x16 MFMAs; operands are
// dequantized while being stored to LDS, so each element is converted once
// per workgroup rather than once per wave.
#include <cmath>

#include "device_common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace mxq {
namespace {

constexpr int BK = 64;
constexpr int RB = BK * 2;    // LDS bytes per row (16-bit elements)
constexpr int CH = RB / 16;   // 16-byte chunks per LDS row
constexpr int kSlabTiles = 32;

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

enum : int { K_NV = 0, K_MX8 = 1, K_MX4 = 2, K_I4 = 3, K_BF = 4 };

struct DqParams {
  GemmP g;
  const float* a_gp;   // NVFP4 tensor scale of a
  const float* w_gp;   // NVFP4 tensor scale of w
  float* part;         // split K: fp32 partial sums [splits][M][N], else null
  int kt_split;        // K-tiles per split (blockIdx.y selects the split)
};

__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 32 NVFP4 codes (16 bytes) with block scales s0 (elements 0-15) and s1
// (16-31) -> 64 bytes of fp16 (FP16=true) or bf16 values.
template <bool FP16>
__device__ __forceinline__ void dq_fp4_nv(const uint4& c, float s0, float s1, uint4 out[4]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[16];
  if constexpr (FP16) {
    const v2h h0 = {(_Float16)s0, (_Float16)s0}, h1 = {(_Float16)s1, (_Float16)s1};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const v2h sc = (k < 2) ? h0 : h1;
      o[4 * k + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 0) * sc);
      o[4 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 1) * sc);
      o[4 * k + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 2) * sc);
      o[4 * k + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 3) * sc);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float sc = (k < 2) ? s0 : s1;
      const v2f f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], 1.0f, 0);
      const v2f f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], 1.0f, 1);
      const v2f f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], 1.0f, 2);
      const v2f f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], 1.0f, 3);
      o[4 * k + 0] = pack_hi16(f0.x * sc, f0.y * sc);   // exact products, exact truncation
      o[4 * k + 1] = pack_hi16(f1.x * sc, f1.y * sc);
      o[4 * k + 2] = pack_hi16(f2.x * sc, f2.y * sc);
      o[4 * k + 3] = pack_hi16(f3.x * sc, f3.y * sc);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
}

// 32 MXFP4 codes with one E8M0 scale (a power of two) -> bf16.
__device__ __forceinline__ void dq_fp4_mx(const uint4& c, float sc, uint4 out[4]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[4 * k + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[k], sc, 0));
    o[4 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[k], sc, 1));
    o[4 * k + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[k], sc, 2));
    o[4 * k + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[k], sc, 3));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
}

// 32 int4 codes (two's complement nibbles) -> 32 bf16 integers.
__device__ __forceinline__ void dq_int4(const uint4& c, uint4 out[4]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[16];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // sign-extend each nibble with an arithmetic shift
      const float lo = (float)((int)(w[k] << (28 - 8 * j)) >> 28);
      const float hi = (float)((int)(w[k] << (24 - 8 * j)) >> 28);
      o[4 * k + j] = pack_hi16(lo, hi);
    }
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
}

// 16 E4M3 codes with one E8M0 scale -> bf16 (32 bytes).
__device__ __forceinline__ void dq_fp8_mx(const uint4& c, float sc, uint4 out[2]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], sc, false));
    o[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], sc, true));
  }
  out[0] = make_uint4(o[0], o[1], o[2], o[3]);
  out[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// Exponent bias of an MX activation operand: a block with E8M0 code c is
// dequantized with the fp32 scale 2**(c - 127 + B), a normal float for every
// code, so every dequantized value is a normal bf16 (B = 10 for MXFP8, whose
// values reach down to 2**-9, 2 for MXFP4); the epilogue multiplies by 2**-B,
// exactly.  MXFP8 blocks then need c <= 236 (amax below 2**117), MXFP4 blocks
// c <= 250 (amax below 2**126).
template <int K> constexpr int mx_bias() { return K == K_MX8 ? 10 : K == K_MX4 ? 2 : 0; }

template <int K>
__device__ __forceinline__ float e8m0_f32(uint32_t code) {
  return __uint_as_float((code + (uint32_t)mx_bias<K>()) << 23);
}

// A thread's staged 4-bit chunk of one K-tile: 32 codes and their scales.
struct Fp4Data {
  uint4 r;
  uint32_t s;
};

// Loader of one 4-bit operand (A or W): a 16-byte chunk of 32 codes per
// thread per K-tile, plus its block scales.
template <int KIND>
struct Fp4Loader {
  const uint8_t* code;
  const uint8_t* scl;
  bool ok;
  int fc;
  __device__ void init(const uint8_t* base, int64_t ld, const uint8_t* sbase, int64_t lds, int row,
                       int nrows, int fc_) {
    fc = fc_;
    ok = row < nrows;
    code = base + (int64_t)(ok ? row : 0) * ld + fc * 16;
    scl = sbase + (int64_t)(ok ? row : 0) * lds;
  }
  __device__ void load(int kt, Fp4Data& d) const {
    d.r = ok ? *reinterpret_cast<const uint4*>(code + (int64_t)kt * 32) : make_uint4(0, 0, 0, 0);
    if constexpr (KIND == K_NV) d.s = *reinterpret_cast<const uint32_t*>(scl + kt * 4);  // 4 x E4M3
    else if constexpr (KIND == K_MX4) d.s = scl[kt * 2 + fc];                            // E8M0
  }
  // Implicit im2col: K-tile kc of the channel row of the pixel `shift` rows
  // away, or zero codes and scales when that pixel is outside the image.
  __device__ void load_conv(int kc, int64_t shift, int64_t ld, int64_t lds, bool in,
                            Fp4Data& d) const {
    d.r = (ok && in) ? *reinterpret_cast<const uint4*>(code + shift * ld + (int64_t)kc * 32)
                     : make_uint4(0, 0, 0, 0);
    const uint8_t* sp = in ? scl + shift * lds : scl;
    uint32_t v = 0;
    if constexpr (KIND == K_NV) v = *reinterpret_cast<const uint32_t*>(sp + kc * 4);
    else if constexpr (KIND == K_MX4) v = sp[kc * 2 + fc];
    d.s = in ? v : 0u;
  }
  template <bool FP16>
  __device__ void convert(const Fp4Data& d, uint4 o[4]) const {
    if constexpr (KIND == K_NV) {
      // the lane's two E4M3 block scales, decoded exactly by the hardware
      // FP8 convert (a power-of-two scale of 1)
      const v2f s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d.s >> (16 * fc), 1.0f, false);
      dq_fp4_nv<FP16>(d.r, s.x, s.y, o);
    } else if constexpr (KIND == K_MX4) {
      dq_fp4_mx(d.r, e8m0_f32<K_MX4>(d.s), o);
    } else {
      dq_int4(d.r, o);
    }
  }
};

template <int AK, int WK, bool LR, bool CONV, bool DEEP, bool SLAB>
__device__ __forceinline__ void dq_body(const DqParams& dp) {
  const GemmP& p = dp.g;
  constexpr bool FP16 = (AK == K_NV && WK == K_NV);
  constexpr bool I4 = (WK == K_I4);
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * RB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * RB];

  const int tile = remap_tile(blockIdx.x, p.tiles_m * p.tiles_n);
  const int m0 = (tile / p.tiles_n) * BM, n0 = (tile % p.tiles_n) * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, half = lane >> 5;
  // this workgroup's K-tiles: all of them, or one split's share
  const int kt0 = dp.part ? blockIdx.y * dp.kt_split : 0;
  const int KT = dp.part ? min(p.K / BK, kt0 + dp.kt_split) : p.K / BK;

  const int fr = tid >> 1, fc = tid & 1;      // 4-bit operands: row, 32-element chunk
  Fp4Loader<WK> wl;
  wl.init(p.w, p.ldw, p.ws, p.ldws, n0 + fr, p.N, fc);
  Fp4Loader<(AK == K_MX8 || AK == K_BF) ? K_MX4 : AK> al;   // 4-bit activations only
  if constexpr (AK != K_MX8 && AK != K_BF) al.init(p.a, p.lda, p.as, p.ldas, m0 + fr, p.M, fc);
  // bf16 activations: four 16-byte chunks (8 elements each) per thread,
  // copied to LDS unchanged.
  int rbf[4], cbf[4];
  const uint8_t* a_bf[4];
  bool a_okbf[4];
  if constexpr (AK == K_BF) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + i * kThreads;
      rbf[i] = q >> 3;
      cbf[i] = q & 7;
      a_okbf[i] = (m0 + rbf[i]) < p.M;
      a_bf[i] = p.a + (int64_t)(a_okbf[i] ? m0 + rbf[i] : 0) * p.lda + cbf[i] * 16;
    }
  }
  // E4M3 activations: two 16-byte chunks (16 elements each) per thread.
  int ar8[2], ac8[2];
  bool a_ok8[2];
  const uint8_t* a_code8[2];
  const uint8_t* a_scl8[2];
  if constexpr (AK == K_MX8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + i * kThreads;
      ar8[i] = q >> 2;
      ac8[i] = q & 3;
      a_ok8[i] = (m0 + ar8[i]) < p.M;
      a_code8[i] = p.a + (int64_t)(a_ok8[i] ? m0 + ar8[i] : 0) * p.lda + ac8[i] * 16;
      a_scl8[i] = p.as + (int64_t)(a_ok8[i] ? m0 + ar8[i] : 0) * p.ldas;
    }
  }
  // Implicit im2col: pixel coordinates of this thread's activation rows.
  uint32_t cv_m[2] = {0u, 0u};   // taps inside the image (conv_mask)
  ConvDiv cv_div{};
  if constexpr (CONV) {
    cv_div = conv_div(p, BK);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = AK == K_MX8 ? m0 + ar8[i] : m0 + fr;
      cv_m[i] = conv_mask(p, row < p.M ? row : 0);
    }
  }
  // INT4 weights: this lane's output columns' fp32 block scales.
  const float* sw_row[2];
  float2 sw[2];
  if constexpr (I4) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = n0 + wn * 64 + j * 32 + l32;
      sw_row[j] = reinterpret_cast<const float*>(p.ws + (int64_t)(c < p.N ? c : p.N - 1) * p.ldws);
    }
  }

  // One K-tile's global loads, held in registers until stored to LDS (two
  // tiles are in flight: each has a full K-tile of compute to land).
  struct Stage {
    Fp4Data w;        // weight codes and scales
    Fp4Data a;        // 4-bit activations
    uint4 a16[4];     // bf16 activations (4 chunks) or E4M3 (2 chunks)
    uint32_t a8s[2];  // E4M3 activations' E8M0 scales
    float2 sc[2];     // INT4 weights' block scales of this lane's columns
  };
  auto gload = [&](int kt, Stage& S) __attribute__((always_inline)) {
    wl.load(kt, S.w);
    if constexpr (CONV) {
      const ConvTap tp = conv_tap(p, cv_div, kt);
      if constexpr (AK == K_MX8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bool in = conv_inside(cv_m[i], tp);
          S.a16[i] = (a_ok8[i] && in)
                         ? *reinterpret_cast<const uint4*>(a_code8[i] + (int64_t)tp.shift * p.lda +
                                                           (int64_t)tp.kc * 64)
                         : make_uint4(0, 0, 0, 0);
          const uint8_t* sp = in ? a_scl8[i] + (int64_t)tp.shift * p.ldas : a_scl8[i];
          const uint32_t v = sp[tp.kc * 2 + (ac8[i] >> 1)];
          S.a8s[i] = in ? v : 0u;
        }
      } else {
        al.load_conv(tp.kc, tp.shift, p.lda, p.ldas, conv_inside(cv_m[0], tp), S.a);
      }
    } else if constexpr (AK == K_MX8) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        S.a16[i] = a_ok8[i] ? *reinterpret_cast<const uint4*>(a_code8[i] + (int64_t)kt * 64)
                            : make_uint4(0, 0, 0, 0);
        S.a8s[i] = a_scl8[i][kt * 2 + (ac8[i] >> 1)];
      }
    } else if constexpr (AK == K_BF) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S.a16[i] = a_okbf[i] ? *reinterpret_cast<const uint4*>(a_bf[i] + (int64_t)kt * 128)
                             : make_uint4(0, 0, 0, 0);
    } else {
      al.load(kt, S.a);
    }
    if constexpr (I4) {
#pragma unroll
      for (int j = 0; j < 2; ++j) S.sc[j] = *reinterpret_cast<const float2*>(sw_row[j] + kt * 2);
    }
  };
  auto lstore = [&](int buf, const Stage& S) __attribute__((always_inline)) {
    uint4 o[4];
    wl.template convert<FP16>(S.w, o);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = fc * 4 + k;
      *reinterpret_cast<uint4*>(&sB[buf][fr * RB + ((c ^ swz<CH>(fr)) * 16)]) = o[k];
    }
    if constexpr (AK == K_BF) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(&sA[buf][rbf[i] * RB + ((cbf[i] ^ swz<CH>(rbf[i])) * 16)]) = S.a16[i];
    } else if constexpr (AK == K_MX8) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint4 o2[2];
        dq_fp8_mx(S.a16[i], e8m0_f32<K_MX8>(S.a8s[i]), o2);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int c = ac8[i] * 2 + k;
          *reinterpret_cast<uint4*>(&sA[buf][ar8[i] * RB + ((c ^ swz<CH>(ar8[i])) * 16)]) = o2[k];
        }
      }
    } else {
      al.template convert<FP16>(S.a, o);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = fc * 4 + k;
        *reinterpret_cast<uint4*>(&sA[buf][fr * RB + ((c ^ swz<CH>(fr)) * 16)]) = o[k];
      }
    }
  };
  auto mfma = [&](const uint4& a, const uint4& b, const v16f& c) -> v16f {
    if constexpr (FP16)
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                    __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                     __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  };

  // column tiles of this wave that hold any of the N columns (wave-uniform)
  const int live_j = n0 + wn * 64 + 32 < p.N ? 2 : (n0 + wn * 64 < p.N ? 1 : 0);
  // fp32 slabs of kSlabTiles K-tiles (S21) where a workgroup's share of K
  // is longer than one slab
  v16f acc[2][2], tot[SLAB ? 2 : 1][SLAB ? 2 : 1];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  if constexpr (SLAB) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) tot[i][j] = v16f{};
  }

  // Multiply K-tile kt from LDS buffer (kt - kt0) & 1 (INT4 block scales in sw).
  auto mma = [&](int kt) __attribute__((always_inline)) {
    const int buf = (kt - kt0) & 1;
    uint4 af[BK / 16][2], bf[BK / 16][2];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = ks * 2 + half;
        const int r = wm * 64 + i * 32 + l32;
        af[ks][i] = *reinterpret_cast<const uint4*>(&sA[buf][r * RB + ((c ^ swz<CH>(r)) * 16)]);
        const int rb = wn * 64 + i * 32 + l32;
        bf[ks][i] = *reinterpret_cast<const uint4*>(&sB[buf][rb * RB + ((c ^ swz<CH>(rb)) * 16)]);
      }
    if constexpr (I4) {
      // two 32-element blocks per K-tile: exact block partials, then the fp32
      // block scale of each output column.  A wave skips its column tiles
      // that lie wholly past N (narrow weight groups: 20 INT4 rows).
      auto blocks = [&](int nj) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              if (j >= nj) continue;
              v16f part = mfma(af[2 * b][i], bf[2 * b][j], v16f{});
              part = mfma(af[2 * b + 1][i], bf[2 * b + 1][j], part);
              const float s = b == 0 ? sw[j].x : sw[j].y;
#pragma unroll
              for (int q = 0; q < 16; ++q) acc[i][j][q] = fmaf(part[q], s, acc[i][j][q]);
            }
      };
      if (live_j == 2) blocks(2);
      else if (live_j == 1) blocks(1);
    } else {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma(af[ks][i], bf[ks][j], acc[i][j]);
    }
    if constexpr (SLAB) {
      if ((kt - kt0 + 1) % kSlabTiles == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            tot[i][j] += acc[i][j];
            acc[i][j] = v16f{};
          }
      }
    }
  };

  if constexpr (DEEP) {
    // Two K-tiles in flight.  At K-tile kt the stage `mine` is free (its
    // INT4 scales are copied first) and `nxt` holds K-tile kt + 1: load
    // K-tile kt + 2 into `mine`, multiply K-tile kt, store K-tile kt + 1.
    // The load is unconditional (the last ones reload K-tile KT - 1): one
    // under a branch would make the compiler wait for it before the store.
    auto iter = [&](int kt, Stage& mine, Stage& nxt) __attribute__((always_inline)) {
      if constexpr (I4) {
#pragma unroll
        for (int j = 0; j < 2; ++j) sw[j] = mine.sc[j];
      }
      gload(kt + 2 < KT ? kt + 2 : KT - 1, mine);
      mma(kt);
      if (kt + 1 < KT) lstore(((kt - kt0) & 1) ^ 1, nxt);
      __syncthreads();
    };
    Stage sg0, sg1;
    gload(kt0, sg0);
    gload(kt0 + 1 < KT ? kt0 + 1 : KT - 1, sg1);
    lstore(0, sg0);
    __syncthreads();
    for (int kt = kt0; kt < KT; kt += 2) {
      iter(kt, sg0, sg1);
      if (kt + 1 < KT) iter(kt + 1, sg1, sg0);
    }
  } else {
    // One K-tile in flight: load K-tile kt + 1, multiply K-tile kt, store.
    Stage sg;
    gload(kt0, sg);
    lstore(0, sg);
    __syncthreads();
    for (int kt = kt0; kt < KT; ++kt) {
      if constexpr (I4) {
#pragma unroll
        for (int j = 0; j < 2; ++j) sw[j] = sg.sc[j];
      }
      if (kt + 1 < KT) gload(kt + 1, sg);
      mma(kt);
      if (kt + 1 < KT) lstore(((kt - kt0) & 1) ^ 1, sg);
      __syncthreads();
    }
  }
  if constexpr (SLAB) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] += tot[i][j];
  }
  if (dp.part) {
    // split K: this split's fp32 sums (C layout: lane column l32, rows
    // 8(q/4) + 4*half + q%4 of each 32x32 tile); launch_splitk_reduce finishes
    float* part = dp.part + (int64_t)blockIdx.y * p.M * p.N;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = m0 + wm * 64 + i * 32 + 8 * (q / 4) + 4 * half + q % 4;
          if (row < p.M) part[(int64_t)row * p.N + n] = acc[i][j][q];
        }
    }
    return;
  }
  // undo the MX exponent bias (a power of two), then the NVFP4 tensor scales
  float alpha = __uint_as_float((uint32_t)(127 - mx_bias<AK>()) << 23);
  if constexpr (AK == K_NV) alpha *= *dp.a_gp;
  if constexpr (WK == K_NV) alpha *= *dp.w_gp;
  epilogue<LR>(p, acc, alpha, m0, n0, wm, wn, lane);
}

// Without slabs (a share of K of at most kSlabTiles K-tiles) the registers
// allow two workgroups per compute unit.
template <int AK, int WK, bool LR, bool SLAB>
__global__ __launch_bounds__(kThreads, SLAB ? 1 : 2) void gemm_dq_kernel(DqParams dp) {
  dq_body<AK, WK, LR, false, false, SLAB>(dp);
}

// Grids of at most one workgroup per compute unit (narrow weight groups,
// split K) are bound by load latency: two K-tiles in flight.
template <int AK, int WK, bool LR>
__global__ __launch_bounds__(kThreads) void gemm_dq_deep_kernel(DqParams dp) {
  dq_body<AK, WK, LR, false, true, true>(dp);
}

// The same GEMM with the activation operand read as the implicit im2col of a
// 3x3 convolution.
template <int AK, int WK, bool DEEP, bool SLAB>
__global__ __launch_bounds__(kThreads, SLAB ? 1 : 2) void conv_dq_kernel(DqParams dp) {
  dq_body<AK, WK, false, true, DEEP, SLAB>(dp);
}

template <int AK, int WK>
hipError_t dispatch(bool lr, dim3 grid, const DqParams& p, hipStream_t s) {
  // at most one workgroup per compute unit: two K-tiles in flight
  const bool deep = (int64_t)grid.x * grid.y <= 256;
  const int share = p.part ? p.kt_split : p.g.K / BK;   // K-tiles per workgroup
  const bool slab = share > kSlabTiles;
  if (p.g.cv_c > 0) {
    // implicit im2col of a quantized input (none for bf16 input)
    if constexpr (AK == K_BF) return hipErrorInvalidValue;
    else if (deep) conv_dq_kernel<AK, WK, true, true><<<grid, kThreads, 0, s>>>(p);
    else if (slab) conv_dq_kernel<AK, WK, false, true><<<grid, kThreads, 0, s>>>(p);
    else conv_dq_kernel<AK, WK, false, false><<<grid, kThreads, 0, s>>>(p);
  } else if (deep) {
    if (lr) gemm_dq_deep_kernel<AK, WK, true><<<grid, kThreads, 0, s>>>(p);
    else gemm_dq_deep_kernel<AK, WK, false><<<grid, kThreads, 0, s>>>(p);
  } else {
    if (slab) {
      if (lr) gemm_dq_kernel<AK, WK, true, true><<<grid, kThreads, 0, s>>>(p);
      else gemm_dq_kernel<AK, WK, false, true><<<grid, kThreads, 0, s>>>(p);
    } else {
      if (lr) gemm_dq_kernel<AK, WK, true, false><<<grid, kThreads, 0, s>>>(p);
      else gemm_dq_kernel<AK, WK, false, false><<<grid, kThreads, 0, s>>>(p);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.part) return e;
  return launch_splitk_reduce(p.g, p.part, (int)grid.y, AK == K_NV ? p.a_gp : nullptr,
                              std::ldexp(1.0f, -mx_bias<AK>()), s);
}

template <int AK>
hipError_t dispatch_w(int w_fmt, bool lr, dim3 grid, const DqParams& p, hipStream_t s) {
  if (w_fmt != FMT_INT4) return hipErrorInvalidValue;   // MX/NVFP4 weights: gemm_dqp.hip
  return dispatch<AK, K_I4>(lr, grid, p, s);
}

}  // namespace

constexpr int kMaxSplits = 16;

// K splits of an M x N x K problem: narrow weight groups (at most 128
// output tiles) split K to fill the chip (about 256 workgroups, at most 4
// splits), and further, up to 16 splits, into shares of at most kSlabTiles
// K-tiles: those run without fp32 slabs at two workgroups per CU.
int dq_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t kt = K / BK;
  if (tiles <= 0 || tiles > 128 || kt < 2) return 1;
  int64_t s = 256 / tiles;
  s = s > 4 ? 4 : s;
  const int64_t s_slab = (kt + kSlabTiles - 1) / kSlabTiles;
  if (s_slab > s) s = s_slab < kMaxSplits ? s_slab : kMaxSplits;
  return (int)(s < kt ? s : kt);
}

// Workspace for any K: narrow groups may take up to kMaxSplits fp32 partials.
int64_t gemm_dq_workspace(int64_t M, int64_t N) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles <= 0 || tiles > 128) return 0;
  return (int64_t)kMaxSplits * M * N * 4;
}

hipError_t launch_gemm_dq(const GemmArgs& a, hipStream_t s) {
  DqParams dp;
  GemmP& p = dp.g;
  p.a = a.a_codes; p.lda = a.lda; p.as = a.a_scales; p.ldas = a.ld_as;
  p.w = a.w_codes; p.ldw = a.ldw; p.ws = a.w_scales; p.ldws = a.ld_ws;
  p.M = (int)a.M; p.N = (int)a.N; p.K = (int)a.K;
  p.tiles_m = (int)((a.M + BM - 1) / BM);
  p.tiles_n = (int)((a.N + BN - 1) / BN);
  p.col_map = a.col_map;
  p.u = a.u; p.ld_u = a.ld_u; p.l2t = a.l2t; p.rank = a.rank;
  p.bias = a.bias;
  p.out = a.out; p.ld_out = a.ld_out; p.n_out = (int)a.n_out;
  p.cv_h = (int)a.cv_h; p.cv_w = (int)a.cv_w; p.cv_c = (int)a.cv_c;
  dp.a_gp = a.a_g;
  dp.w_gp = a.w_g;
  dp.part = nullptr;
  dp.kt_split = 0;
  const bool lr = a.rank > 0;
  // Too few tiles to fill the chip (narrow weight groups): split K over
  // blockIdx.y into fp32 partials in the workspace, then sum them in split
  // order (deterministic) in a second kernel.  Not with the low-rank branch.
  // A smaller workspace takes as many splits as fit.
  int splits = lr ? 1 : dq_splits(a.M, a.N, a.K);
  const int64_t per_split = a.M * a.N * 4;
  if (splits > 1 && a.ws && per_split > 0) {
    const int64_t fit = a.ws_bytes / per_split;
    if (fit < splits) splits = (int)fit;
  } else {
    splits = 1;
  }
  if (splits > 1) {
    const int kt = (int)(a.K / BK);
    dp.kt_split = (kt + splits - 1) / splits;
    dp.part = a.ws;
  }
  const dim3 grid(p.tiles_m * p.tiles_n, dp.part ? (unsigned)((a.K / BK + dp.kt_split - 1) / dp.kt_split) : 1u);
  switch (a.a_fmt) {
    case FMT_NVFP4: return dispatch_w<K_NV>(a.w_fmt, lr, grid, dp, s);
    case FMT_MXFP8: return dispatch_w<K_MX8>(a.w_fmt, lr, grid, dp, s);
    case FMT_MXFP4: return dispatch_w<K_MX4>(a.w_fmt, lr, grid, dp, s);
    case FMT_BF16: return dispatch_w<K_BF>(a.w_fmt, lr, grid, dp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mxq
