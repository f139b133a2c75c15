// Block-scaled GEMM on the gfx950 scaled MFMA for MXFP4 activations x MXFP4
// weights: y = RN_bf16(Q(a) Q(w)^T [+ u L2] [+ bias]).
//
// The 4-bit weight x 4-bit activation product is the layer's one dense
// contraction (Nunchaku article, "main explanation": W4A4 speeds up the
// denoising loop; the 16-bit low-rank branch is added to the same output).
// v_mfma_scale_f32_32x32x64_f8f6f4 consumes E2M1 codes directly and applies
// one E8M0 scale per lane per 32 K-values, which is exactly the MX block
// (Microscaling FP4 summary: power-of-two MXFP4 scales), so codes and scales
// go from HBM to the matrix core with no conversion.  For E2M1 x E2M1 its
// dot products are exact before the fp32 accumulation (measured).
//
// Operand layout (checked on gfx950): lane l of a 32x32x64 step holds row
// l % 32 and the 32 E2M1 codes K = 32*(l/32) + [0,32), i.e. 16 bytes; its
// scale register supplies the E8M0 of that row's K-block l/32, the byte
// chosen by op_sel.
//
// Organisation:
//  * workgroup tile (32*TM*WGM) x (64*TN), waves in a WGM x 2 grid (4 or 8
//    waves), each wave (32*TM) x (32*TN) = TM*TN MFMA tiles; K-tile 256
//    (four MFMA K-steps), so every row of a tile contributes one whole
//    128-byte line per K-tile (64-byte half lines take about 1.5x as long
//    to stream at full occupancy);
//  * code tiles stream into a 2-stage LDS ring with direct global->LDS
//    loads one K-tile ahead of the MFMAs (no register staging); each lane's
//    load address is chosen so the bytes land in the XOR-swizzled slot the
//    fragment reads expect;
//  * scales stream two K-tiles at a time (16 contiguous bytes of each row,
//    one 16-byte piece per lane where alignment and K allow, else four
//    dwords) into a 2-buffer ring of their own: per-K-tile 8-byte pieces
//    from every row cost as many cache-line requests as the codes;
//  * one barrier per K-tile; a K-tile's fragments are read at the start of
//    its step and consumed in K-step order while the next K-tile streams in;
//  * the MFMAs compute D^T = W A^T (weight fragment first), so each lane ends
//    up holding four consecutive output columns of one row;
//  * the low-rank term u L2 is accumulated before the main loop, while the
//    first K-tile streams in (only the sum's order changes);
//  * past 16 K-tiles (K > 4096) the fp32 chains are flushed into a second
//    accumulator every 8 K-tiles (small tiles only, for the registers).
#include "device_common.h"
#include "gemm_common.h"
#include "gemm_pipe.h"
#include "kernels.h"

namespace mxq {
namespace {

constexpr int BK = 256;           // K per tile
constexpr int RB = BK / 2;        // bytes per row per K-tile (E2M1)
constexpr int CH = RB / 16;       // 16-byte chunks per row
constexpr int KS = BK / 64;       // MFMA K-steps per K-tile
constexpr int SB = BK / 32;       // scale bytes per row per K-tile
constexpr int kSlab = 8;          // K-tiles per fp32 slab when slabbing

// Whole-tile staged epilogue (no column map; 16-byte aligned output rows):
// each wave writes its accumulators (+ bias, bf16) into the LDS image of the
// workgroup tile -- rows [0, TBM/2) in `lo`, the rest in `hi` -- then every
// thread stores 16-byte pieces of whole tile rows with non-temporal stores.
// Accumulator layout (D^T = W A^T): lane l of MFMA tile (i, j) holds row
// i*32 + l%32 and columns j*32 + 8g + 4(l/32) + [0, 4) at acc[i][j][4g..4g+3].
template <int TM, int TN, int WGM, int STAGE>
__device__ __forceinline__ void epilogue_wg(const GemmP& p, v16f (&acc)[TM][TN], int m0, int n0,
                                            int wm, int wn, int lane, uint8_t* lo, uint8_t* hi) {
  constexpr int TBM = 32 * TM * WGM, TBN = 64 * TN, NT = 128 * WGM;
  constexpr int WRS = TBN * 2 + 16, CPR = TBN / 8;   // row stride; 16-byte pieces per row
  const int l32 = lane & 31, half = lane >> 5;
  const int n_lim = p.N < p.n_out ? p.N : p.n_out;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = wm * 32 * TM + i * 32 + l32;
    uint8_t* row = (r < TBM / 2 ? lo + r * WRS : hi + (r - TBM / 2) * WRS);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = wn * 32 * TN + j * 32 + 8 * g + 4 * half;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int nn = n0 + c + e;
          v[e] = acc[i][j][4 * g + e] + ((p.bias && nn < n_lim) ? bf16_bits_to_f32(p.bias[nn]) : 0.f);
        }
        uint2 pk;
        pk.x = pack_bf16_rne(v[0], v[1]);
        pk.y = pack_bf16_rne(v[2], v[3]);
        *reinterpret_cast<uint2*>(row + c * 2) = pk;
      }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < TBM * CPR; idx += NT) {
    const int r = idx / CPR, ch = idx % CPR;
    const uint8_t* src = (r < TBM / 2 ? lo + r * WRS : hi + (r - TBM / 2) * WRS) + ch * 16;
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    const int row = m0 + r, n = n0 + ch * 8;
    if (row >= p.M) continue;
    uint16_t* o = p.out + (int64_t)row * p.ld_out + n;
    if (n + 8 <= n_lim) {
      __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(o));
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < n_lim) o[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

template <int TM, int TN, int WGM, bool SLAB, bool LR, bool VSC>
__global__ __launch_bounds__(128 * WGM, 1) void gemm_mx_kernel(GemmP p, int gm) {
  constexpr int NW = 2 * WGM;                      // waves: WGM (rows) x 2 (columns)
  constexpr int TBM = 32 * TM * WGM, TBN = 64 * TN;
  constexpr int A_STAGE = TBM * RB, W_STAGE = TBN * RB;
  constexpr bool PAD = (TBM * CH / 64) % NW != 0 || (TBN * CH / 64) % NW != 0;
  constexpr int STAGE = A_STAGE + W_STAGE + (PAD ? 1024 : 0);
  // scale groups: G K-tiles (one step pair), SROW bytes per row, a buffer
  // per group in flight
  constexpr int G = 2;
  constexpr int SROW = G * SB, SGRP = (TBM + TBN) * SROW;
  static_assert(((TBM + TBN) * SROW) % 1024 == 0, "whole 64-lane scale loads");
  // two separate code stages: reads of one are visibly independent of the
  // loads in flight into the other, so the compiler adds no wait for them;
  // scales are read right after the step's wait, with no load outstanding
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t scl[2 * SGRP + 1024];   // + spare-load pad

  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, gm, tm, tn);
  const int m0 = tm * TBM, n0 = tn * TBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, half = lane >> 5;
  const int KT = (p.K + BK - 1) / BK;
  // a K that is an odd multiple of 128 leaves the last K-tile half full
  const int last_ch = (p.K % BK) ? (p.K % BK) / 32 : CH;

  // Byte offsets within a stage of this lane's fragment and scale reads.  At
  // K-step s the lane supplies K = 64s + 32*half + [0, 32) of its row, i.e.
  // chunk 2s + half, stored at chunk (2s + half) ^ swz(row).  Every row the
  // lane reads is l32 plus a multiple of 32, all with the same swizzle, so
  // one register per K-step serves all of them (the rows differ by constant
  // offsets).
  const uint8_t* zsrc = zero_src();
  const int swl = swz<CH>(l32);
  uint32_t a_base[KS], w_base[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint32_t c = ((2 * s + half) ^ swl) * 16;
    a_base[s] = (wm * 32 * TM + l32) * RB + c;
    w_base[s] = A_STAGE + (wn * 32 * TN + l32) * RB + c;
  }
  const uint32_t sa_base = (wm * 32 * TM + l32) * SROW;
  const uint32_t sw_base = (TBM + wn * 32 * TN + l32) * SROW;

  auto issue = [&](int kt, uint8_t* st) __attribute__((always_inline)) {
    const bool past = kt >= KT;   // past the end of K: a tile of zeros
    kt = past ? KT - 1 : kt;
    const int lim = kt == KT - 1 ? last_ch : CH;
    uint8_t* pad = st + A_STAGE + W_STAGE;
    issue_tile<TBM, RB, NW>(p.a, p.lda, m0, p.M, kt, st, wave, lane, zsrc, past, pad, lim);
    issue_tile<TBN, RB, NW>(p.w, p.ldw, n0, p.N, kt, st + A_STAGE, wave, lane, zsrc, past, pad, lim);
  };
  // Scale group g (K-tiles gG .. gG+G-1) into buffer g % 2: rows of A, then
  // rows of W, SROW bytes each.  VSC (16-byte aligned scale rows, K a
  // multiple of G K-tiles): one 16-byte piece per lane, else one dword per
  // lane.  Pieces past the row's scales read zeros; rows past M or N re-read
  // the last row.  Every wave issues the same number of loads, so the code
  // has no branch; spare ones copy zeros into a pad.
  const int srow_bytes = p.K / 32;
  auto issue_scales = [&](int g) __attribute__((always_inline)) {
    constexpr int PB = VSC ? 16 : 4;   // bytes per lane
    constexpr int PER = SROW / PB, LOADS = SGRP / (64 * PB);
    uint8_t* buf = scl + (g & 1) * SGRP;
    const int k0 = g * SROW;   // byte offset of the group within a scale row
#pragma unroll
    for (int t = 0; t < (LOADS + NW - 1) / NW; ++t) {
      const int idx = t * NW + wave;
      const bool real = LOADS % NW == 0 || idx < LOADS;
      const int slot = (real ? idx : 0) * 64 + lane, r = slot / PER, q = slot % PER;
      // both candidate rows from scalar parameters, then a select (a
      // per-lane choice between parameters would read them from memory)
      const int ra = min(m0 + r, p.M - 1), rw = max(min(n0 + r - TBM, p.N - 1), 0);
      const uint8_t* pa = p.as + (int64_t)ra * p.ldas;
      const uint8_t* pw = p.ws + (int64_t)rw * p.ldws;
      const uint8_t* src = (r < TBM ? pa : pw) + k0 + q * PB;
      src = real && k0 + q * PB < srow_bytes ? src : zsrc;
      uint8_t* dst = real ? buf + idx * 64 * PB : scl + 2 * SGRP;
      if constexpr (VSC) __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
      else __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 4, 0, 0);
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

  // Read the K-tile's fragments and scales from stage `st` and multiply,
  // the fragments of K-step s+1 read while the MFMAs of K-step s run.  The
  // scale dword d of a row holds the E8M0 of K-blocks 4d .. 4d+3; the lane's
  // byte for K-step s (block 2s + half) sits at byte 2(s%2) of dword s/2
  // after shifting by 8*half.
  uint2 sa2[TM], sw2[TN];
  auto read_scales = [&](int kt) __attribute__((always_inline)) {
    const uint8_t* buf = scl + ((kt / G) & 1) * SGRP + (kt % G) * SB;
#pragma unroll
    for (int i = 0; i < TM; ++i) sa2[i] = *reinterpret_cast<const uint2*>(buf + sa_base + i * 32 * SROW);
#pragma unroll
    for (int j = 0; j < TN; ++j) sw2[j] = *reinterpret_cast<const uint2*>(buf + sw_base + j * 32 * SROW);
  };
  auto compute = [&](const uint8_t* st) __attribute__((always_inline)) {
    v4i fa[2][TM], fw[2][TN];
    auto frag = [&](int s, int b) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fw[b][j] = *reinterpret_cast<const v4i*>(st + w_base[s] + j * 32 * RB);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[b][i] = *reinterpret_cast<const v4i*>(st + a_base[s] + i * 32 * RB);
    };
    frag(0, 0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) frag(s + 1, (s + 1) & 1);
      uint32_t sa[TM], sw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) sa[i] = (s < 2 ? sa2[i].x : sa2[i].y) >> (8 * half);
#pragma unroll
      for (int j = 0; j < TN; ++j) sw[j] = (s < 2 ? sw2[j].x : sw2[j].y) >> (8 * half);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          // E2M1 operands use the low four dwords of the 8-dword register
          const v4i& w4 = fw[s & 1][j];
          const v4i& a4 = fa[s & 1][i];
          const v8i wv = __builtin_shufflevector(w4, w4, 0, 1, 2, 3, -1, -1, -1, -1);
          const v8i av = __builtin_shufflevector(a4, a4, 0, 1, 2, 3, -1, -1, -1, -1);
          if (s % 2 == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                wv, av, acc[i][j], 4, 4, 0, (int)sw[j], 0, (int)sa[i]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                wv, av, acc[i][j], 4, 4, 2, (int)sw[j], 2, (int)sa[i]);
        }
    }
  };

  // One K-tile (tile t lives in stage t % 2): wait until K-tile kt has
  // landed and read its scales (their group landed at least one step
  // earlier), barrier (every wave is done reading stage (kt+1) % 2, the one
  // K-tile kt-1 lived in, and the scale buffer of the previous group), load
  // K-tile kt+1 (and, at a group's first K-tile, the next scale group), and
  // multiply K-tile kt.  The loop runs a whole number of 2-step groups with
  // no branch around the MFMAs (keeping the accumulators in place); K-tiles
  // past the end are loaded as zeros.
  constexpr int NT = tile_loads<TBM, RB, NW>() + tile_loads<TBN, RB, NW>();   // per wave per K-tile
  constexpr int N_MFMA = KS * TM * TN;
  constexpr int N_DS0 = TM + TN;                  // K-step 0
  constexpr int N_DS1 = (KS - 1) * (TM + TN);     // K-steps 1 .. KS-1
  // K-tile 1 is issued in the prologue, so the first step waits only for
  // K-tile 0 and issues no codes
  auto step = [&](int kt, const uint8_t* st_cur, uint8_t* st_nxt, bool even, bool first) __attribute__((always_inline)) {
    // nothing of the previous step sinks below the wait
    __builtin_amdgcn_sched_barrier(0);
    if (first) wait_vmcnt<NT>();
    else wait_vmcnt<0>();
    read_scales(kt);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");   // no LDS read moves above the barrier
    if (!first) issue(kt + 1, st_nxt);
    if (even) issue_scales(kt / G + 1);
    compute(st_cur);
    // K-step 0 first; then one MFMA, one fragment read (running a K-step
    // ahead) and one of the next K-tile's loads at a time
    __builtin_amdgcn_sched_group_barrier(0x100, N_DS0, 0);
#pragma unroll
    for (int k = 0; k < N_MFMA; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (k < N_DS1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (k < NT) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    if constexpr (SLAB) {
      if (kt < KT && (kt + 1) % kSlab == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            tot[i][j] += acc[i][j];
            acc[i][j] = v16f{};
          }
      }
    }
  };

  // Prologue: K-tile 0, scale group 0, the low-rank operands (up to 32
  // ranks), then K-tile 1 into the other stage.  The low-rank branch goes
  // into the accumulators first, its MFMAs running while K-tile 1 is in
  // flight (the loads complete in issue order, so waiting for all but
  // K-tile 1's NT loads covers everything before them).
  issue(0, st0);
  issue_scales(0);
  LrFrag<TM, TN> lrf;
  const int lr_nt = LR ? (p.rank / 16 < 2 ? p.rank / 16 : 2) : 0;
  if constexpr (LR) lr_load<TM, TN>(p, lrf, 0, lr_nt, m0 + wm * 32 * TM, n0 + wn * 32 * TN, lane);
  issue(1, st1);
  wait_vmcnt<NT>();
  if constexpr (LR) {
    lr_mma<TM, TN>(lrf, lr_nt, acc);
    // ranks past the first 32 (rare): their own loads and waits
    for (int t0 = 2; t0 < p.rank / 16; t0 += 2) {
      LrFrag<TM, TN> f;
      const int nt = p.rank / 16 - t0 < 2 ? p.rank / 16 - t0 : 2;
      lr_load<TM, TN>(p, f, t0, nt, m0 + wm * 32 * TM, n0 + wn * 32 * TN, lane);
      lr_mma<TM, TN>(f, nt, acc);
    }
  }
  __builtin_amdgcn_s_barrier();   // K-tile 0 and scale group 0 visible to every wave
  step(0, st0, st1, true, true);
  step(1, st1, st0, false, false);
  for (int kt = 2; kt < KT; kt += 2) {
    step(kt, st0, st1, true, false);
    step(kt + 1, st1, st0, false, false);
  }
  wait_vmcnt<0>();   // the zero loads issued past the end
  if constexpr (SLAB) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] += tot[i][j];
  }
  // the stages are free once every wave is past its last fragment read;
  // each wave stages its output rows in its own slice of one of them
  wait_lgkmcnt0();
  __syncthreads();
  // The workgroup's whole output tile goes through LDS (its upper half of
  // rows in one stage, the lower half in the other) and leaves as 16-byte
  // pieces of whole rows, so every 128-byte line of the output is written
  // by one store instruction (a per-wave staging splits the lines that
  // straddle two waves' columns).
  constexpr int WRS = TBN * 2 + 16;            // LDS bytes per staged row (padded)
  if constexpr ((TBM / 2) * WRS <= STAGE) {
    if (!p.col_map && (p.ld_out & 7) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 15) == 0) {
      epilogue_wg<TM, TN, WGM, STAGE>(p, acc, m0, n0, wm, wn, lane, st0, st1);
      return;
    }
  }
  constexpr int RG = 32 * (TN * 64 + 16), SL = STAGE / RG;   // staging slices per stage
  static_assert(2 * SL >= NW, "a staging slice per wave");
  uint8_t* region = (wave / SL == 0 ? st0 : st1) + (wave % SL) * RG;
  epilogue_tr<false, TM, TN>(p, acc, 1.0f, m0 + wm * 32 * TM, n0 + wn * 32 * TN, lane, region);
}

template <int TM, int TN, int WGM, bool SLAB>
hipError_t launch_cfg(bool lr, GemmP p, hipStream_t s) {
  p.tiles_m = (p.M + 32 * TM * WGM - 1) / (32 * TM * WGM);
  p.tiles_n = (p.N + 64 * TN - 1) / (64 * TN);
  const int tiles = p.tiles_m * p.tiles_n;
  // tile-rows per group: one XCD's share (tiles / 8) as a near-square block
  int gm = 1;
  while (gm * 2 <= p.tiles_m && gm * 2 * gm * 2 <= (tiles + 7) / 8) gm *= 2;
  // 16-byte scale pieces need 16-byte aligned scale rows in both operands
  // and K a multiple of two K-tiles (whole 16-byte groups)
  const bool vsc = p.ldas % 16 == 0 && p.ldws % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(p.as) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(p.ws) % 16 == 0 && p.K % (2 * BK) == 0;
  const dim3 grid(tiles);
  if (lr && vsc) gemm_mx_kernel<TM, TN, WGM, SLAB, true, true><<<grid, 128 * WGM, 0, s>>>(p, gm);
  else if (lr) gemm_mx_kernel<TM, TN, WGM, SLAB, true, false><<<grid, 128 * WGM, 0, s>>>(p, gm);
  else if (vsc) gemm_mx_kernel<TM, TN, WGM, SLAB, false, true><<<grid, 128 * WGM, 0, s>>>(p, gm);
  else gemm_mx_kernel<TM, TN, WGM, SLAB, false, false><<<grid, 128 * WGM, 0, s>>>(p, gm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t s) {
  GemmP p;
  p.a = a.a_codes; p.lda = a.lda; p.as = a.a_scales; p.ldas = a.ld_as;
  p.w = a.w_codes; p.ldw = a.ldw; p.ws = a.w_scales; p.ldws = a.ld_ws;
  p.M = (int)a.M; p.N = (int)a.N; p.K = (int)a.K;
  p.col_map = a.col_map;
  p.u = a.u; p.ld_u = a.ld_u; p.l2t = a.l2t; p.rank = a.rank;
  p.bias = a.bias;
  p.out = a.out; p.ld_out = a.ld_out; p.n_out = (int)a.n_out;
  p.cv_h = (int)a.cv_h; p.cv_w = (int)a.cv_w; p.cv_c = (int)a.cv_c;
  const bool lr = a.rank > 0;
  if (a.K > 4096) return launch_cfg<2, 2, 2, true>(lr, p, s);
  // Large tiles move the fewest bytes per MFMA; pick the one whose tile count
  // fills the 256 compute units in the fewest rounds, per unit of tile work.
  const int64_t cu = 256;
  auto rounds = [&](int tbm, int tbn) __attribute__((always_inline)) {
    const int64_t t = ((a.M + tbm - 1) / tbm) * ((a.N + tbn - 1) / tbn);
    return (t + cu - 1) / cu;
  };
  // (work per tile in 64x64 output blocks, x10)
  const int64_t c43 = rounds(256, 192) * 12 * 10;
  const int64_t c44 = rounds(256, 256) * 16 * 10;
  const int64_t c22 = rounds(128, 128) * 4 * 16;    // small tiles run ~60% as efficiently
  if (c22 < c43 && c22 < c44) {
    // a grid of fewer than 128 such tiles leaves most compute units idle and
    // each workgroup latency-bound: 64x64 tiles (four times as many
    // workgroups) finish sooner (256 x 1152 x 1152: 10.2 -> 6.5 us)
    if (((a.M + 127) / 128) * ((a.N + 127) / 128) < 128) return launch_cfg<1, 1, 2, false>(lr, p, s);
    return launch_cfg<2, 2, 2, false>(lr, p, s);
  }
  // 256-row tiles run eight waves (4 x 2, two per SIMD): one wave's waits
  // overlap the other's MFMAs
  if (c44 < c43) return launch_cfg<2, 4, 4, false>(lr, p, s);
  return launch_cfg<2, 3, 4, false>(lr, p, s);
}

}  // namespace mxq
