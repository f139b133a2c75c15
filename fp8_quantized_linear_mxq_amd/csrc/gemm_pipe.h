// Building blocks of the pipelined GEMM kernels: direct global->LDS tile
// loads into a ring of stages, explicit memory-counter waits, a grouped
// tile order, and the epilogue for the transposed accumulator layout.
#pragma once

#include "device_common.h"
#include "gemm_common.h"

namespace mxq {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// 16 zero bytes (one copy per code object): the source of every load of a
// K-tile past the end of K, so such a tile multiplies to exactly zero and the
// main loop needs no branch.
static __device__ uint8_t g_zero16[16];

// The address of g_zero16 held in two VGPRs for the life of a kernel.  The
// symbol is reached through the GOT, and left to itself the compiler reloads
// it with a scalar load inside the main loop; a scalar load in flight turns
// every LDS wait in the loop into a full drain (LDS reads and scalar loads
// share one counter, and scalar loads may return out of order), so each
// MFMA group would wait for the fragment reads just issued for the next step.
__device__ __forceinline__ const uint8_t* zero_src() {
  const uint64_t a = reinterpret_cast<uint64_t>(g_zero16);
  uint32_t lo = (uint32_t)a, hi = (uint32_t)(a >> 32);
  asm volatile("" : "+v"(lo));
  asm volatile("" : "+v"(hi));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// Direct loads of one operand tile (ROWS rows x RB bytes of K-tile kt) into
// an LDS stage.  The tile is ROWS*CH/64 64-lane instructions, dealt to the NW
// waves round-robin; slot L (16 bytes) of the stage holds row L / CH, physical
// chunk L % CH, which is logical chunk (L % CH) ^ swz(row): each lane fetches
// the global chunk that belongs in its slot.  Rows past the operand's end
// re-read its last row (their results are never stored); with `zero` set every
// lane reads zeros.  Every wave issues tile_loads<ROWS, RB, NW>() loads; where
// the count does not divide evenly the spare ones copy zeros into `pad` (1 KB),
// so each wave's memory counter advances by the same amount.  Chunks at or
// past logical chunk `lim` (a K-tile cut short by the end of K) read zeros.
template <int ROWS, int RB, int NW>
constexpr int tile_loads() { return (ROWS * RB / 1024 + NW - 1) / NW; }

template <int ROWS, int RB, int NW = 4>
__device__ __forceinline__ void issue_tile(const uint8_t* base, int64_t ld, int row0, int nrows,
                                           int kt, uint8_t* stage, int wave, int lane,
                                           const uint8_t* zsrc, bool zero = false,
                                           uint8_t* pad = nullptr, int lim = RB / 16) {
  constexpr int CH = RB / 16;
  constexpr int TOTAL = ROWS * CH / 64;
  static_assert(ROWS * CH % 64 == 0, "tile must split into whole 64-lane loads");
#pragma unroll
  for (int t = 0; t < tile_loads<ROWS, RB, NW>(); ++t) {
    const int idx = t * NW + wave;
    const bool real = (TOTAL % NW == 0) || idx < TOTAL;
    const int slot0 = (real ? idx : 0) * 64;
    const int L = slot0 + lane;
    const int r = L / CH, pc = L % CH;
    int grow = row0 + r;
    grow = grow < nrows ? grow : nrows - 1;
    const int lc = pc ^ swz<CH>(r);
    const uint8_t* src = base + (int64_t)grow * ld + (int64_t)kt * RB + lc * 16;
    const bool cut = lim < RB / 16 && lc >= lim;
    src = (zero || !real || cut) ? zsrc : src;
    uint8_t* dst = real ? stage + slot0 * 16 : pad;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
  }
}

// Direct loads of one K-tile's block-scale bytes of both operands, one dword
// per lane: TBM rows of A (SBA bytes each), then TBN rows of W (SBW bytes
// each); lanes past the end re-read a valid dword into padding; with `zero`
// set every lane reads zeros, and so do dwords at or past dword `lim_a` of
// an A row or `lim_w` of a W row (a K-tile cut short by the end of K); zeros
// come from zsrc (zero_src()).  Issues
// ceil((TBM*SBA + TBN*SBW) / (256*NW)) loads per wave.
template <int TBM, int SBA, int TBN, int SBW, int NW = 4>
__device__ __forceinline__ void issue_scale_tile(const GemmP& p, int m0, int n0, int kt,
                                                 uint8_t* region, int wave, int lane,
                                                 const uint8_t* zsrc,
                                                 bool zero = false, int lim_a = SBA / 4,
                                                 int lim_w = SBW / 4) {
  constexpr int DA = TBM * SBA / 4, D = DA + TBN * SBW / 4;
  constexpr int PERW = (D + 64 * NW - 1) / (64 * NW);
  constexpr int QA = SBA >= 4 ? SBA / 4 : 1;   // dwords per A row (A may have no scales)
#pragma unroll
  for (int t = 0; t < PERW; ++t) {
    const int slot0 = (t * NW + wave) * 64;
    const int d = slot0 + lane;
    const uint8_t* src;
    bool cut = false;
    if (d < DA) {
      int r = m0 + d / QA;
      r = r < p.M ? r : p.M - 1;
      cut = lim_a < SBA / 4 && d % QA >= lim_a;
      src = p.as + (int64_t)r * p.ldas + kt * SBA + (d % QA) * 4;
    } else if (d < D) {
      const int e = d - DA;
      int r = n0 + e / (SBW / 4);
      r = r < p.N ? r : p.N - 1;
      cut = lim_w < SBW / 4 && e % (SBW / 4) >= lim_w;
      src = p.ws + (int64_t)r * p.ldws + kt * SBW + (e % (SBW / 4)) * 4;
    } else {
      src = SBA ? p.as + (int64_t)(m0 < p.M ? m0 : p.M - 1) * p.ldas + kt * SBA : zsrc;
    }
    src = (zero || cut) ? zsrc : src;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(region + slot0 * 4), 4, 0, 0);
  }
}

template <int TBM, int SBA, int TBN, int SBW, int NW = 4>
constexpr int scale_region_bytes() {
  return ((TBM * SBA / 4 + TBN * SBW / 4 + 64 * NW - 1) / (64 * NW)) * 256 * NW;
}

// Workgroup -> output tile.  Workgroups are dealt to the 8 XCDs round-robin;
// each XCD gets a contiguous range of tile ids, walked GM tile-rows at a
// time so the A and W bands one XCD streams stay small enough for its L2.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int gm, int& tm,
                                            int& tn) {
  const int t = remap_tile(bid, tiles_m * tiles_n);
  const int per_group = gm * tiles_n;
  const int g = t / per_group, r = t % per_group;
  const int rows = (tiles_m - g * gm) < gm ? (tiles_m - g * gm) : gm;
  tm = g * gm + r % rows;
  tn = r / rows;
}

// Two floats -> packed bf16, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t){a, b}, v2bf_t));
}

// The low-rank branch u L2 added into the transposed accumulators (the
// MFMAs compute D^T = W A^T: lane l of tile (i, j) holds output row
// row0 + i*32 + l%32 and columns col0 + j*32 + 8g + 4(l/32) + [0,4)).  u is
// split into bf16 halves u_hi + u_lo (residual <= 2**-17 |u|): two K = rank
// passes of bf16 MFMAs per 16 ranks.  L2 is read by output column (through
// the column map).  The loads (lr_load, up to 32 ranks held in registers)
// and the MFMAs (lr_mma) are separate steps, so a kernel can issue other
// loads in between; add_lowrank does both for any rank.
template <int TI, int TN>
struct LrFrag {
  float4 u[2][TI][2];   // ranks 16t + 8*half + [0, 8) of the lane's rows
  uint4 l[2][TN];       // L2 rows (bf16) of the lane's output columns
};

template <int TI, int TN>
__device__ __forceinline__ void lr_load(const GemmP& p, LrFrag<TI, TN>& f, int t0, int nt,
                                        int row0, int col0, int lane) {
  const int l32 = lane & 31, half = lane >> 5;
  // output columns first (a map lookup only when there is a map), so the L2
  // addresses wait on nothing but these lookups
  int col[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) col[j] = col0 + j * 32 + l32;
  if (p.col_map) {
#pragma unroll
    for (int j = 0; j < TN; ++j) col[j] = col[j] < p.N ? p.col_map[col[j]] : 0;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) col[j] = (col[j] < p.N || p.col_map) && col[j] >= 0 && col[j] < p.n_out ? col[j] : 0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t >= nt) break;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      int row = row0 + i * 32 + l32;
      row = row < p.M ? row : p.M - 1;
      const float* up = p.u + (int64_t)row * p.ld_u + (t0 + t) * 16 + half * 8;
      f.u[t][i][0] = *reinterpret_cast<const float4*>(up);
      f.u[t][i][1] = *reinterpret_cast<const float4*>(up + 4);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
      f.l[t][j] = *reinterpret_cast<const uint4*>(p.l2t + (int64_t)col[j] * p.rank + (t0 + t) * 16 + half * 8);
  }
}

template <int TI, int TN>
__device__ __forceinline__ void lr_mma(const LrFrag<TI, TN>& f, int nt, v16f (&acc)[TI][TN]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t >= nt) break;
    v8bf ufr_h[TI], ufr_l[TI];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const float4 f0 = f.u[t][i][0], f1 = f.u[t][i][1];
      const float v[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = f32_to_bf16_bits(v[e]);
        lo[e] = f32_to_bf16_bits(v[e] - bf16_bits_to_f32(hi[e]));
      }
      ufr_h[i] = __builtin_bit_cast(v8bf, make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                                                     hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)));
      ufr_l[i] = __builtin_bit_cast(v8bf, make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16),
                                                     lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const v8bf lf = __builtin_bit_cast(v8bf, f.l[t][j]);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf, ufr_h[i], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf, ufr_l[i], acc[i][j], 0, 0, 0);
      }
    }
  }
}

template <int TI, int TN>
__device__ __forceinline__ void add_lowrank(const GemmP& p, v16f (&acc)[TI][TN], int row0, int col0,
                                            int lane) {
  for (int t0 = 0; t0 < p.rank / 16; t0 += 2) {
    LrFrag<TI, TN> f;
    const int nt = p.rank / 16 - t0 < 2 ? p.rank / 16 - t0 : 2;
    lr_load<TI, TN>(p, f, t0, nt, row0, col0, lane);
    lr_mma<TI, TN>(f, nt, acc);
  }
}

// Epilogue for the transposed accumulator layout: scales by alpha, adds the
// low-rank branch (LR), the bias, and applies the column map.  `lds_region`
// (32 * (TN * 64 + 16) bytes private to the wave, or null) enables the
// staged row-wise stores.
template <bool LR, int TI, int TN>
__device__ __forceinline__ void epilogue_tr(const GemmP& p, v16f (&acc)[TI][TN], float alpha,
                                            int row0, int col0, int lane,
                                            uint8_t* lds_region = nullptr) {
  const int l32 = lane & 31, half = lane >> 5;
  if (alpha != 1.0f) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] *= alpha;
  }
  if constexpr (LR) add_lowrank<TI, TN>(p, acc, row0, col0, lane);
  // stores: without a column map and with a 16-byte aligned output, each
  // 32-row tile goes through the wave's LDS region (row-major) and leaves as
  // 16-byte pieces of whole rows; otherwise each lane stores its quads
  // directly (the four columns of a quad are shared by its TI rows, so their
  // map entries and bias are fetched once per quad).
  const int n_lim = p.N < p.n_out ? p.N : p.n_out;
  const bool staged = lds_region && !p.col_map && (p.ld_out & 7) == 0 &&
                      (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
  const bool vec = !p.col_map && (p.ld_out & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.out) & 7) == 0;
  if (staged) {
    constexpr int RS = TN * 64 + 16;        // LDS bytes per staged row (padded)
    constexpr int CPR = TN * 4;             // 16-byte pieces per row
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int nn = col0 + j * 32 + 8 * g + 4 * half + e;
            v[e] = acc[i][j][4 * g + e] + ((p.bias && nn < n_lim) ? bf16_bits_to_f32(p.bias[nn]) : 0.f);
          }
          uint2 pk;
          pk.x = pack_bf16_rne(v[0], v[1]);
          pk.y = pack_bf16_rne(v[2], v[3]);
          *reinterpret_cast<uint2*>(lds_region + l32 * RS + (j * 32 + 8 * g + 4 * half) * 2) = pk;
        }
#pragma unroll
      for (int t = 0; t < 32 * CPR / 64; ++t) {
        const int idx = t * 64 + lane;
        const int r = idx / CPR, ch = idx % CPR;
        const uint4 v = *reinterpret_cast<const uint4*>(lds_region + r * RS + ch * 16);
        const int row = row0 + i * 32 + r, n = col0 + ch * 8;
        if (row < p.M) {
          uint16_t* o = p.out + (int64_t)row * p.ld_out + n;
          if (n + 8 <= n_lim) {
            // streaming store: the output is not read again by this kernel
            // (5-6% faster GEMMs than cached stores at 4096 x 3072 / 4608)
            __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(o));
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < n_lim) o[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = col0 + j * 32 + 8 * g + 4 * half;
      int c[4];
      float b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int nn = n + e;
        c[e] = nn < p.N ? (p.col_map ? p.col_map[nn] : nn) : -1;
        if (c[e] >= p.n_out) c[e] = -1;
        b[e] = (p.bias && c[e] >= 0) ? bf16_bits_to_f32(p.bias[c[e]]) : 0.f;
      }
      const bool full = vec && n + 3 < n_lim;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = row0 + i * 32 + l32;
        if (row >= p.M) continue;
        uint16_t* orow = p.out + (int64_t)row * p.ld_out;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] + b[e];
        if (full) {
          uint2 pk;
          pk.x = pack_bf16_rne(v[0], v[1]);
          pk.y = pack_bf16_rne(v[2], v[3]);
          *reinterpret_cast<uint2*>(orow + n) = pk;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c[e] >= 0) orow[c[e]] = (uint16_t)f32_to_bf16_bits(v[e]);
        }
      }
    }
  }
}

}  // namespace mxq
