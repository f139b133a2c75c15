// Pipelined exact-dequant GEMM for MX/NVFP4 weights: every (activation,
// weight) pair with A in {MXFP8, NVFP4, MXFP4} and W in {MXFP4, NVFP4} except
// MXFP4 x MXFP4, which has its own scaled-MFMA kernel; also unquantized bf16
// activations (4-bit weights, 16-bit activations), which skip the activation
// dequantization.
//
// Arithmetic (why 16-bit): on gfx950 the MFMAs that take E4M3 operands keep
// only about 15 bits below the largest product of each dot product, which
// cannot meet the layer's 1e-5 * sum|a w| bound on heavy-tailed activations,
// while the 16-bit MFMAs round like fp32.  Each code times its block scale is
// exact in a 16-bit float: E4M3 x E8M0 and E2M1 x E8M0 have <= 4 significant
// bits (bf16 for the E8M0 range), E2M1 x E4M3 (NVFP4) <= 6 bits within
// [2**-10, 2688] (fp16 when both operands are NVFP4, bf16 otherwise).  NVFP4
// tensor scales multiply the accumulator in the epilogue.
//
// Organisation (the same pipeline as the MXFP4 kernel):
//  * workgroup tile (32*TM*WGM) x (32*TN*WGN), WGM*WGN waves in a WGM x WGN
//    grid (four, or eight for 256-row tiles), each wave (32*TM) x (32*TN):
//    every dequantized fragment feeds TN (activation) or TM (weight) MFMAs.
//    An NVFP4 fragment dequantized to bf16 costs four converts, eight
//    multiplies and four packs against an MX fragment's four converts (a
//    bf16 activation fragment costs none), so the operand that is dearer to
//    dequantize gets the longer side of the wave tile: tall tiles (TM > TN)
//    for NVFP4 weights against MX or bf16 activations and for MXFP4 weights
//    against bf16 activations, wide ones for NVFP4 activations against
//    MXFP4 weights;
//  * raw code and scale tiles (4-bit codes are a quarter, 8-bit codes half
//    the bytes of 16-bit tiles) stream into a 3-stage LDS ring with direct
//    global->LDS loads two K-tiles ahead of the MFMAs;
//  * inside a 128-wide K-tile the reduction index is permuted identically for
//    both operands: lane half h supplies K = 64h + 8ks + [0, 8) at MFMA step
//    ks, so a lane's fragments for the whole K-tile are one contiguous run of
//    its row (2-4 16-byte LDS reads) and every fragment lies in one scale
//    block; the sum's terms are only reordered;
//  * a step reads its K-tile's activation runs one 16-byte chunk ahead of
//    the MFMAs that use them (few registers, so 128-row wave tiles fit); the
//    loop is branch-free (tiles past the end of K load as zeros);
//  * the MFMAs compute D^T = W A^T and the output leaves through LDS as
//    16-byte pieces of whole rows.
#include "device_common.h"
#include "gemm_common.h"
#include "gemm_pipe.h"
#include "kernels.h"

namespace mxq {
namespace {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));

enum : int { K_NV = 0, K_MX8 = 1, K_MX4 = 2, K_BF = 3 };

constexpr int BK = 128;
constexpr int kSlab = 6;   // K-tiles (8 MFMA steps each) per fp32 slab when slabbing

template <int K> constexpr int row_bytes() { return K == K_BF ? 256 : K == K_MX8 ? 128 : 64; }
template <int K> constexpr int scale_bytes() { return K == K_BF ? 0 : K == K_NV ? 8 : 4; }

struct DqpParams {
  GemmP g;
  const float* a_gp;   // NVFP4 tensor scale of a
  const float* w_gp;   // NVFP4 tensor scale of w
  int gm;              // tile-rows per group of the tile order
};

__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Exponent bias of an MX operand in this route: a block with E8M0 code c is
// dequantized with the fp32 scale 2**(c - 127 + B), so that every code gives
// a normal fp32 scale (2**-127 is a subnormal the converts do not apply
// exactly) and every dequantized value is a normal bf16 (E4M3 values reach
// down to 2**-9, E2M1 to 2**-1): B = 10 for MXFP8, 2 for MXFP4.  The
// epilogue multiplies by 2**-(B_a + B_w), exactly.  The price is the top
// codes: a value must stay below bf16's 2**128, so MXFP8 blocks need
// c <= 236 (block amax below 2**117) and MXFP4 blocks c <= 250 (amax below
// 2**126).
template <int K> constexpr int mx_bias() { return K == K_MX8 ? 10 : K == K_MX4 ? 2 : 0; }

template <int K>
__device__ __forceinline__ float e8m0_scale(uint32_t code) {
  return __uint_as_float((code + (uint32_t)mx_bias<K>()) << 23);
}

// The lane's block scales of a K-tile, one value per group of MFMA steps:
// MX: steps 0-3 and 4-7 (two 32-blocks), NVFP4: steps 2q, 2q+1 (16-blocks).
template <int K, bool FP16>
struct Scales {
  float s[K == K_NV ? 4 : 2];
};

template <int K, bool FP16>
__device__ __forceinline__ Scales<K, FP16> lane_scales(uint32_t dw, int half) {
  Scales<K, FP16> r;
  if constexpr (K == K_BF) {
    r.s[0] = r.s[1] = 1.0f;   // no scales
  } else if constexpr (K == K_NV) {
    // dword `half` of the row's 8 scale bytes: 16-blocks 4h .. 4h+3.  The
    // hardware FP8 converts decode the four E4M3 codes exactly (a power-of-
    // two scale of 1), two per instruction, in place of a bit-field decode
    // of about seven instructions per code.
    const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(dw, 1.0f, false);
    const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(dw, 1.0f, true);
    r.s[0] = lo.x;
    r.s[1] = lo.y;
    r.s[2] = hi.x;
    r.s[3] = hi.y;
  } else {
    // bytes 2h, 2h+1 of the row's 4 scale bytes: 32-blocks 2h, 2h+1
    const uint32_t b = dw >> (16 * half);
    r.s[0] = e8m0_scale<K>(b & 0xFFu);
    r.s[1] = e8m0_scale<K>((b >> 8) & 0xFFu);
  }
  return r;
}

// Dequantize MFMA step ks (8 elements) of a lane's raw run to 16-bit values.
template <int K, bool FP16>
__device__ __forceinline__ uint4 dq(const uint32_t* raw, int ks, const Scales<K, FP16>& sc) {
  if constexpr (K == K_BF) {
    return make_uint4(raw[4 * ks], raw[4 * ks + 1], raw[4 * ks + 2], raw[4 * ks + 3]);
  } else if constexpr (K == K_MX8) {
    const float s = sc.s[ks >> 2];
    const uint32_t d0 = raw[2 * ks], d1 = raw[2 * ks + 1];
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, s, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, s, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, s, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, s, true)));
  } else if constexpr (K == K_MX4) {
    const float s = sc.s[ks >> 2];
    const uint32_t d = raw[ks];
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3)));
  } else {
    const float s = sc.s[ks >> 1];
    const uint32_t d = raw[ks];
    if constexpr (FP16) {
      const v2h sh = {(_Float16)s, (_Float16)s};
      return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * sh),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * sh),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * sh),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * sh));
    } else {
      // products of <= 6 significant bits: truncating the fp32 product to
      // its top 16 bits is exact
      const v2f f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
      const v2f f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
      const v2f f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
      const v2f f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
      return make_uint4(pack_hi16(f0.x * s, f0.y * s), pack_hi16(f1.x * s, f1.y * s),
                        pack_hi16(f2.x * s, f2.y * s), pack_hi16(f3.x * s, f3.y * s));
    }
  }
}

template <int AK, int WK, int TM, int TN, int WGM, bool SLAB, bool LR, bool CONV, int WGN>
__device__ __forceinline__ void dqp_body(const DqpParams& dp) {
  const GemmP& p = dp.g;
  constexpr bool FP16 = (AK == K_NV && WK == K_NV);
  constexpr int NW = WGM * WGN;   // waves: WGM (rows) x WGN (columns)
  constexpr int TBM = 32 * TM * WGM, TBN = 32 * TN * WGN;
  constexpr int A_RB = row_bytes<AK>(), W_RB = row_bytes<WK>();
  constexpr int A_CH = A_RB / 16, W_CH = W_RB / 16;
  constexpr int SBA = scale_bytes<AK>(), SBW = scale_bytes<WK>();
  constexpr int A_STAGE = TBM * A_RB, W_STAGE = TBN * W_RB;
  constexpr int S_STAGE = scale_region_bytes<TBM, SBA, TBN, SBW, NW>();
  constexpr bool PAD = (TBM * A_CH / 64) % NW != 0 || (TBN * W_CH / 64) % NW != 0;
  constexpr int STAGE = A_STAGE + W_STAGE + S_STAGE + (PAD ? 1024 : 0);
  constexpr int NT = tile_loads<TBM, A_RB, NW>() + tile_loads<TBN, W_RB, NW>() +
                     S_STAGE / (256 * NW);   // loads per wave per K-tile
  constexpr int A_DW = A_RB / 8, W_DW = W_RB / 8;   // dwords of a lane's run per K-tile
  static_assert(2 * NT < 64, "vmcnt range");
  // three separate arrays: reads of one stage are visibly independent of the
  // loads in flight into the others, so the compiler adds no wait for them
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];

  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, dp.gm, tm, tn);
  const int m0 = tm * TBM, n0 = tn * TBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, half = lane >> 5;
  const int KT = p.K / BK;

  // Byte offsets within a stage of this lane's fragment and scale reads.
  // Every row the lane reads is l32 plus a multiple of 32, and the swizzle
  // depends on the row's low bits only, so one register per 16-byte chunk
  // serves all row tiles (they differ by constant offsets).
  uint32_t a_base[A_DW / 4], w_base[W_DW / 4];
#pragma unroll
  for (int t = 0; t < A_DW / 4; ++t) {
    const int c = half * (A_CH / 2) + t;
    a_base[t] = (wm * 32 * TM + l32) * A_RB + ((c ^ swz<A_CH>(l32)) * 16);
  }
#pragma unroll
  for (int t = 0; t < W_DW / 4; ++t) {
    const int c = half * (W_CH / 2) + t;
    w_base[t] = A_STAGE + (wn * 32 * TN + l32) * W_RB + ((c ^ swz<W_CH>(l32)) * 16);
  }
  const uint32_t sa_base = A_STAGE + W_STAGE + (wm * 32 * TM + l32) * SBA + (SBA == 8 ? 4 * half : 0);
  const uint32_t sw_base =
      A_STAGE + W_STAGE + TBM * SBA + (wn * 32 * TN + l32) * SBW + (SBW == 8 ? 4 * half : 0);

  // Implicit im2col: the row address and pixel of each of this lane's
  // activation code loads and activation scale loads, fixed for the whole
  // loop (the lane-to-slot map of issue_tile / issue_scale_tile); each K-tile
  // adds its tap's row shift and reads zeros where the shifted pixel lies
  // outside the image.  Loads that carry no row of A never read.
  constexpr int A_LD = tile_loads<TBM, A_RB, NW>();
  constexpr int S_DA = TBM * SBA / 4, S_D = S_DA + TBN * SBW / 4;
  constexpr int S_LD = (S_D + 64 * NW - 1) / (64 * NW);
  const uint8_t* cv_code[CONV ? A_LD : 1];
  uint32_t cv_m[CONV ? A_LD : 1];     // taps inside the image (conv_mask)
  const uint8_t* cv_scl[CONV ? S_LD : 1];
  uint32_t cv_sm[CONV ? S_LD : 1];
  ConvDiv cv_div{};
  if constexpr (CONV) {
    cv_div = conv_div(p, BK);
    constexpr int TOTAL = TBM * A_CH / 64;
#pragma unroll
    for (int t = 0; t < A_LD; ++t) {
      const int idx = t * NW + wave;
      const bool real = (TOTAL % NW == 0) || idx < TOTAL;
      const int L = (real ? idx : 0) * 64 + lane;
      const int r = L / A_CH, lc = (L % A_CH) ^ swz<A_CH>(r);
      const int grow = m0 + r < p.M ? m0 + r : p.M - 1;
      cv_code[t] = p.a + (int64_t)grow * p.lda + lc * 16;
      cv_m[t] = real ? conv_mask(p, grow) : 0u;
    }
#pragma unroll
    for (int t = 0; t < S_LD; ++t) {
      const int d = (t * NW + wave) * 64 + lane;
      const int dd = d < S_DA ? d : 0;
      const int grow = m0 + dd / (SBA / 4) < p.M ? m0 + dd / (SBA / 4) : p.M - 1;
      cv_scl[t] = p.as + (int64_t)grow * p.ldas + (dd % (SBA / 4)) * 4;
      cv_sm[t] = d < S_DA ? conv_mask(p, grow) : 0u;
    }
  }

  const uint8_t* zsrc = zero_src();
  auto issue = [&](int kt, uint8_t* st) __attribute__((always_inline)) {
    const bool past = kt >= KT;   // past the end of K: a tile of zeros
    kt = past ? KT - 1 : kt;
    uint8_t* pad = st + A_STAGE + W_STAGE + S_STAGE;
    if constexpr (CONV) {
      const ConvTap tp = conv_tap(p, cv_div, kt);
      const int64_t off = (int64_t)tp.shift * p.lda + tp.kc * A_RB;
      constexpr int TOTAL = TBM * A_CH / 64;
#pragma unroll
      for (int t = 0; t < A_LD; ++t) {
        const int idx = t * NW + wave;
        const bool real = (TOTAL % NW == 0) || idx < TOTAL;
        const bool in = !past && conv_inside(cv_m[t], tp);
        const uint8_t* src = in ? cv_code[t] + off : zsrc;
        uint8_t* dst = real ? st + idx * 64 * 16 : pad;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
      }
      issue_tile<TBN, W_RB, NW>(p.w, p.ldw, n0, p.N, kt, st + A_STAGE, wave, lane, zsrc, past, pad);
      // scales: activation rows through the tap, weight rows as issue_scale_tile
      const int64_t soff = (int64_t)tp.shift * p.ldas + tp.kc * SBA;
      uint8_t* region = st + A_STAGE + W_STAGE;
#pragma unroll
      for (int t = 0; t < S_LD; ++t) {
        const int slot0 = (t * NW + wave) * 64;
        const int d = slot0 + lane;
        const uint8_t* src;
        if (d < S_DA) {
          src = conv_inside(cv_sm[t], tp) ? cv_scl[t] + soff : zsrc;
        } else if (d < S_D) {
          const int e = d - S_DA;
          int r = n0 + e / (SBW / 4);
          r = r < p.N ? r : p.N - 1;
          src = p.ws + (int64_t)r * p.ldws + kt * SBW + (e % (SBW / 4)) * 4;
        } else {
          src = zsrc;
        }
        src = past ? zsrc : src;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(region + slot0 * 4), 4, 0, 0);
      }
    } else {
      issue_tile<TBM, A_RB, NW>(p.a, p.lda, m0, p.M, kt, st, wave, lane, zsrc, past, pad);
      issue_tile<TBN, W_RB, NW>(p.w, p.ldw, n0, p.N, kt, st + A_STAGE, wave, lane, zsrc, past, pad);
      issue_scale_tile<TBM, SBA, TBN, SBW, NW>(p, m0, n0, kt, st + A_STAGE + W_STAGE, wave, lane,
                                               zsrc, past);
    }
  };

  v16f acc[TM][TN];
  v16f tot[SLAB ? TM : 1][SLAB ? TN : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};
  if constexpr (SLAB) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) tot[i][j] = v16f{};
  }

  // Dequantize and multiply the K-tile in stage `st`.  The weight runs and
  // all scales are read up front; the activation runs are read one 16-byte
  // chunk (A_KS MFMA steps) ahead of their use, so only two chunks per row
  // tile are ever held in registers.
  constexpr int A_NC = A_DW / 4;          // 16-byte chunks per lane run
  constexpr int A_KS = (BK / 16) / A_NC;  // MFMA steps per chunk
  auto compute = [&](const uint8_t* st) __attribute__((always_inline)) {
    uint32_t wraw[TN][W_DW];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int t = 0; t < W_DW / 4; ++t) {
        const uint4 v = *reinterpret_cast<const uint4*>(st + w_base[t] + j * 32 * W_RB);
        wraw[j][4 * t] = v.x; wraw[j][4 * t + 1] = v.y; wraw[j][4 * t + 2] = v.z; wraw[j][4 * t + 3] = v.w;
      }
    Scales<AK, FP16> sa[TM];
    Scales<WK, FP16> sw[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      sa[i] = SBA ? lane_scales<AK, FP16>(*reinterpret_cast<const uint32_t*>(st + sa_base + i * 32 * SBA), half)
                  : lane_scales<AK, FP16>(0u, half);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sw[j] = lane_scales<WK, FP16>(*reinterpret_cast<const uint32_t*>(st + sw_base + j * 32 * SBW), half);
    uint4 ach[2][TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) ach[0][i] = *reinterpret_cast<const uint4*>(st + a_base[0] + i * 32 * A_RB);
#pragma unroll
    for (int c = 0; c < A_NC; ++c) {
      if (c + 1 < A_NC) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          ach[(c + 1) & 1][i] = *reinterpret_cast<const uint4*>(st + a_base[c + 1] + i * 32 * A_RB);
      }
#pragma unroll
      for (int kk = 0; kk < A_KS; ++kk) {
        const int ks = c * A_KS + kk;
        uint4 af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          // the chunk's dwords sit at run positions 4c .. 4c+3
          uint32_t run[A_DW];
          const uint4 v = ach[c & 1][i];
          run[4 * c] = v.x; run[4 * c + 1] = v.y; run[4 * c + 2] = v.z; run[4 * c + 3] = v.w;
          af[i] = dq<AK, FP16>(run, ks, sa[i]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = dq<WK, FP16>(wraw[j], ks, sw[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (FP16)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(v8h, bf[j]), __builtin_bit_cast(v8h, af[i]), acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(v8bf, bf[j]), __builtin_bit_cast(v8bf, af[i]), acc[i][j], 0, 0, 0);
          }
      }
    }
  };

  // One K-tile (tile t lives in stage t % 3): wait until K-tile kt has landed
  // (kt+1 may still be in flight) and this wave's reads are complete, then
  // barrier (every wave is done with stage (kt-1) % 3), load K-tile kt+2
  // into that stage, and dequantize and multiply K-tile kt from its stage.
  auto step = [&](int kt, const uint8_t* st_cur, uint8_t* st_load) __attribute__((always_inline)) {
    wait_vmcnt<NT>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    issue(kt + 2, st_load);
    compute(st_cur);
  };

  // the loop runs a whole number of 3-step groups (slabbing: 6-step groups,
  // each flushed into the second accumulator at its end) with no branch,
  // keeping the accumulators in place; K-tiles past the end load as zeros
  issue(0, st0);
  issue(1, st1);
  if constexpr (SLAB) {
    static_assert(kSlab == 6, "one slab per loop iteration");
    for (int kt = 0; kt < KT; kt += 6) {
      step(kt, st0, st2);
      step(kt + 1, st1, st0);
      step(kt + 2, st2, st1);
      step(kt + 3, st0, st2);
      step(kt + 4, st1, st0);
      step(kt + 5, st2, st1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          tot[i][j] += acc[i][j];
          acc[i][j] = v16f{};
        }
    }
  } else {
    for (int kt = 0; kt < KT; kt += 3) {
      step(kt, st0, st2);
      step(kt + 1, st1, st0);
      step(kt + 2, st2, st1);
    }
  }
  wait_vmcnt<0>();   // the zero loads issued past the end
  if constexpr (SLAB) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] += tot[i][j];
  }
  // undo the MX exponent biases (a power of two), then the NVFP4 tensor scales
  float alpha = __uint_as_float((uint32_t)(127 - mx_bias<AK>() - mx_bias<WK>()) << 23);
  if constexpr (AK == K_NV) alpha *= *dp.a_gp;
  if constexpr (WK == K_NV) alpha *= *dp.w_gp;
  wait_lgkmcnt0();
  __syncthreads();
  constexpr int RG = 32 * (TN * 64 + 16), SL = STAGE / RG;   // staging slices per stage
  static_assert(3 * SL >= NW, "a staging slice per wave");
  uint8_t* region = (wave / SL == 0 ? st0 : wave / SL == 1 ? st1 : st2) + (wave % SL) * RG;
  epilogue_tr<LR, TM, TN>(p, acc, alpha, m0 + wm * 32 * TM, n0 + wn * 32 * TN, lane, region);
}

// Tall wave tiles where the weight fragment is the dearer one to dequantize
// (NVFP4 weights against MX or bf16 activations): 128x128 workgroup tiles as
// 1 x 4 waves of 128 x 32 instead of 2 x 2 of 64 x 64 (0.25 weight and one
// activation fragment per MFMA instead of 0.5 and 0.5), 256x256 as 2 x 4
// waves of 128 x 64 instead of 4 x 2 of 64 x 128.  Wide ones where the
// activation fragment is (NVFP4 activations, MXFP4 weights): 128x128 as
// 4 x 1 waves of 32 x 128 (the 256x256 tile's 64 x 128 waves are wide
// already).
template <int AK, int WK>
constexpr bool tall_waves() { return WK == K_NV && AK != K_NV; }
template <int AK, int WK>
constexpr bool wide_waves() { return AK == K_NV && WK == K_MX4; }

// Slabbed tiles run two workgroups per CU, except with bf16 activations,
// whose three LDS stages take 123 KB.
template <int AK, int WK, int TM, int TN, int WGM, bool SLAB, bool LR, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN, (SLAB && AK != K_BF) ? 2 : 1) void gemm_dqp_kernel(
    DqpParams dp) {
  dqp_body<AK, WK, TM, TN, WGM, SLAB, LR, false, WGN>(dp);
}

// The same GEMM with the activation operand read as the implicit im2col of a
// 3x3 convolution (128x128 tiles, two workgroups per compute unit).
template <int AK, int WK, bool SLAB>
__global__ __launch_bounds__(256, 2) void conv_dqp_kernel(DqpParams dp) {
  if constexpr (tall_waves<AK, WK>()) dqp_body<AK, WK, 4, 1, 1, SLAB, false, true, 4>(dp);
  else if constexpr (wide_waves<AK, WK>()) dqp_body<AK, WK, 1, 4, 4, SLAB, false, true, 1>(dp);
  else dqp_body<AK, WK, 2, 2, 2, SLAB, false, true, 2>(dp);
}

template <int AK, int WK, int TM, int TN, bool SLAB, int WGM = 2, int WGN = 2>
hipError_t launch_cfg(bool lr, DqpParams dp, hipStream_t s) {
  dp.g.tiles_m = (dp.g.M + 32 * TM * WGM - 1) / (32 * TM * WGM);
  dp.g.tiles_n = (dp.g.N + 32 * TN * WGN - 1) / (32 * TN * WGN);
  const int tiles = dp.g.tiles_m * dp.g.tiles_n;
  // tile-rows per group: one XCD's share (tiles / 8) as a near-square block
  dp.gm = 1;
  while (dp.gm * 2 <= dp.g.tiles_m && dp.gm * 2 * dp.gm * 2 <= (tiles + 7) / 8) dp.gm *= 2;
  const dim3 grid(tiles);
  if (lr) gemm_dqp_kernel<AK, WK, TM, TN, WGM, SLAB, true, WGN><<<grid, 64 * WGM * WGN, 0, s>>>(dp);
  else gemm_dqp_kernel<AK, WK, TM, TN, WGM, SLAB, false, WGN><<<grid, 64 * WGM * WGN, 0, s>>>(dp);
  return hipGetLastError();
}

// The 128x128 and 256x256 workgroup tiles in the wave layout the pair takes.
template <int AK, int WK, bool SLAB>
hipError_t launch_128(bool lr, const DqpParams& dp, hipStream_t s) {
  if constexpr (tall_waves<AK, WK>()) return launch_cfg<AK, WK, 4, 1, SLAB, 1, 4>(lr, dp, s);
  else if constexpr (wide_waves<AK, WK>()) return launch_cfg<AK, WK, 1, 4, SLAB, 4, 1>(lr, dp, s);
  else return launch_cfg<AK, WK, 2, 2, SLAB>(lr, dp, s);
}

template <int AK, int WK>
hipError_t launch_256(bool lr, const DqpParams& dp, hipStream_t s) {
  if constexpr (tall_waves<AK, WK>()) return launch_cfg<AK, WK, 4, 2, false, 2, 4>(lr, dp, s);
  else return launch_cfg<AK, WK, 2, 4, false, 4>(lr, dp, s);
}

template <int AK, int WK>
hipError_t launch_conv(DqpParams dp, hipStream_t s) {
  dp.g.tiles_m = (dp.g.M + 127) / 128;
  dp.g.tiles_n = (dp.g.N + 127) / 128;
  const int tiles = dp.g.tiles_m * dp.g.tiles_n;
  dp.gm = 1;
  while (dp.gm * 2 <= dp.g.tiles_m && dp.gm * 2 * dp.gm * 2 <= (tiles + 7) / 8) dp.gm *= 2;
  // long K: fp32 slabs of kSlab K-tiles, as for the plain GEMM
  if (dp.g.K / BK > 32) conv_dqp_kernel<AK, WK, true><<<tiles, 256, 0, s>>>(dp);
  else conv_dqp_kernel<AK, WK, false><<<tiles, 256, 0, s>>>(dp);
  return hipGetLastError();
}

template <int AK, int WK>
hipError_t launch_tiles(bool lr, const DqpParams& dp, hipStream_t s) {
  const int64_t M = dp.g.M, N = dp.g.N;
  // past 32 K-tiles the fp32 chains are flushed into a second accumulator
  // every kSlab K-tiles, which only the small tile has the registers for
  if (dp.g.K / BK > 32) return launch_128<AK, WK, true>(lr, dp, s);
  // Costs in 64x64 output blocks per compute unit over whole rounds of the
  // 256 compute units: the tile that fills them in the fewest rounds per
  // unit of work.  256-row tiles run eight waves (two per SIMD, wave tiles
  // 64 x 96 or 64 x 128); ties go to the wider tile (fewer dequantizations
  // per MFMA).  Short K (under 16 K-tiles) also weighs 128x128 tiles at two
  // workgroups per compute unit (a round of two tiles: 8 blocks), where one
  // tile's pipeline fill and output stores overlap the other's MFMAs; ties
  // go to them.
  const int64_t cu = 256;
  auto rounds = [&](int64_t tbm, int64_t tbn, int64_t slots) {
    const int64_t t = ((M + tbm - 1) / tbm) * ((N + tbn - 1) / tbn);
    return (t + cu * slots - 1) / (cu * slots);
  };
  const int64_t c4 = rounds(256, 256, 1) * 16, c3 = rounds(256, 192, 1) * 12;
  if (dp.g.K / BK < 16) {
    const int64_t c1 = rounds(128, 128, 2) * 8;
    if (c4 < c1 && c4 <= c3) return launch_256<AK, WK>(lr, dp, s);
    if (c3 < c1) return launch_cfg<AK, WK, 2, 3, false, 4>(lr, dp, s);
    return launch_128<AK, WK, false>(lr, dp, s);
  }
  const int64_t c2 = rounds(256, 128, 1) * 8;
  if (c4 <= c3 && c4 <= c2) return launch_256<AK, WK>(lr, dp, s);
  if (c3 <= c2) return launch_cfg<AK, WK, 2, 3, false, 4>(lr, dp, s);
  return launch_cfg<AK, WK, 4, 2, false>(lr, dp, s);
}

template <int AK, int WK>
hipError_t launch_pair(bool lr, const DqpParams& dp, hipStream_t s) {
  if constexpr (AK == K_BF) {
    // 16-bit activation tiles are 256 bytes a row: the 128x128 tile's three
    // stages take 123 KB (one workgroup per CU).  With MXFP4 weights 64x128
    // tiles (75 KB, two per CU; 1 x 4 waves of 64 x 32, since only the
    // weight fragments need converting) are faster (4096x1152x4608: 84 -> 76
    // us with 2 x 2 waves); with NVFP4 weights, whose dequantization is
    // dearer, the taller tile amortizes it over twice the rows and is as fast.
    if (dp.g.cv_c > 0) return hipErrorInvalidValue;
    if (dp.g.K / BK > 32) return launch_128<AK, WK, true>(lr, dp, s);
    if constexpr (WK == K_MX4) return launch_cfg<AK, WK, 2, 1, false, 1, 4>(lr, dp, s);
    else return launch_128<AK, WK, false>(lr, dp, s);
  } else {
    if (dp.g.cv_c > 0) return launch_conv<AK, WK>(dp, s);
    return launch_tiles<AK, WK>(lr, dp, s);
  }
}

template <int AK>
hipError_t launch_w(int w_fmt, bool lr, const DqpParams& dp, hipStream_t s) {
  if (w_fmt == FMT_NVFP4) return launch_pair<AK, K_NV>(lr, dp, s);
  return launch_pair<AK, K_MX4>(lr, dp, s);
}

}  // namespace

hipError_t launch_gemm_dqp(const GemmArgs& a, hipStream_t s) {
  DqpParams dp;
  GemmP& p = dp.g;
  p.a = a.a_codes; p.lda = a.lda; p.as = a.a_scales; p.ldas = a.ld_as;
  p.w = a.w_codes; p.ldw = a.ldw; p.ws = a.w_scales; p.ldws = a.ld_ws;
  p.M = (int)a.M; p.N = (int)a.N; p.K = (int)a.K;
  p.tiles_m = p.tiles_n = 0;
  p.col_map = a.col_map;
  p.u = a.u; p.ld_u = a.ld_u; p.l2t = a.l2t; p.rank = a.rank;
  p.bias = a.bias;
  p.out = a.out; p.ld_out = a.ld_out; p.n_out = (int)a.n_out;
  p.cv_h = (int)a.cv_h; p.cv_w = (int)a.cv_w; p.cv_c = (int)a.cv_c;
  dp.a_gp = a.a_g;
  dp.w_gp = a.w_g;
  const bool lr = a.rank > 0;
  if (a.w_fmt != FMT_NVFP4 && a.w_fmt != FMT_MXFP4) return hipErrorInvalidValue;
  switch (a.a_fmt) {
    case FMT_NVFP4: return launch_w<K_NV>(a.w_fmt, lr, dp, s);
    case FMT_MXFP8: return launch_w<K_MX8>(a.w_fmt, lr, dp, s);
    case FMT_MXFP4: return launch_w<K_MX4>(a.w_fmt, lr, dp, s);
    case FMT_BF16: return launch_w<K_BF>(a.w_fmt, lr, dp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mxq
