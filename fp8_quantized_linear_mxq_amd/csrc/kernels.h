// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

struct LoraDownArgs {
  const uint16_t* x;   // bf16 [rows][ldx]
  int64_t rows, cols, ldx;
  const uint16_t* l1t; // bf16 [rank][cols], or the packed order below
  int rank;
  float* u;            // [rows][ld_u]
  int64_t ld_u;
  bool packed;         // l1t in the fragment order of launch_pack_l1t
};
hipError_t launch_lora_down(const LoraDownArgs& a, hipStream_t s);

// L1^T [rank][cols] (bf16, row stride cols) into the order the fused
// quantize + low-rank kernel reads: 16-byte piece i = ((g NT + t) 4 + j) 64
// + lane holds L1^T[16t + lane % 16][128g + 32(lane / 16) + 8j + [0, 8)],
// NT = rank / 16 (rank a multiple of 16, cols a multiple of 128).
hipError_t launch_pack_l1t(const uint16_t* l1t, int rank, int64_t cols, uint16_t* l1p,
                           hipStream_t s);

struct QuantizeArgs {
  const void* x;
  int dtype;
  int64_t rows, cols, ldx;
  int hadamard_n;
  int fmt;
  uint8_t* codes;
  int64_t ld_codes;
  uint8_t* scales;
  int64_t ld_scales;
  float* tensor_scale_out;          // NVFP4
  const float* static_tensor_scale; // NVFP4, may be null
  float* partials;                  // NVFP4 dynamic: workspace
  const LoraDownArgs* lr;           // optional low-rank down projection (bf16 x)
  unsigned* dbg;                    // debug checks: non-finite flag, else null
  bool nv_two_pass;                 // dynamic NVFP4: skip the one-pass kernel
};

constexpr int kAmaxPartials = 1024;  // NVFP4 phase-1 grid (workspace floats)

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t s);

// Device address and size of the current device's scratch array for the
// allocation-free quantize (the NVFP4 amax partials).
hipError_t quantize_scratch(void** out, size_t* bytes);

// Device address of the non-finite input flag of the current device (the
// debug checks): kernels given it set it to 1 when an input is NaN or Inf.
hipError_t nonfinite_flag_ptr(unsigned** out);



struct GemmArgs {
  int a_fmt, w_fmt;
  const uint8_t* a_codes; int64_t lda;
  const uint8_t* a_scales; int64_t ld_as;
  const float* a_g;
  const uint8_t* w_codes; int64_t ldw;
  const uint8_t* w_scales; int64_t ld_ws;
  const float* w_g;
  int64_t M, N, K;
  const int32_t* col_map;  // may be null
  const float* u; int64_t ld_u;
  const uint16_t* l2t;     // bf16 [n_out][rank]
  int rank;
  const uint16_t* bias;    // bf16 [n_out]
  uint16_t* out; int64_t ld_out; int64_t n_out;
  float* ws; int64_t ws_bytes;   // optional workspace (INT4-row split K)
  // implicit im2col of a 3x3 convolution (0 = plain GEMM): A is the input's
  // [images * cv_h * cv_w][cv_c] pixel rows and K = 9 * cv_c
  int64_t cv_h, cv_w, cv_c;
};
hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t s);
// INT4-row route: K splits for an M x N x K problem (1 = none) and the
// workspace bytes that cover the splits of any K.
int dq_splits(int64_t M, int64_t N, int64_t K);
int64_t gemm_dq_workspace(int64_t M, int64_t N);
hipError_t launch_gemm_dq(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_dqp(const GemmArgs& a, hipStream_t s);

struct SelectArgs {
  const void* w; int dtype;
  int64_t n, k, ldw;
  int cand[4]; int n_cand;
  uint8_t* choice; double* sse; int32_t* perm; int32_t* counts; float* g_out;
  float* partials;   // workspace: kAmaxPartials floats
  double* sse_ws;    // workspace: n * n_cand doubles (when sse is null)
  float* g_ws;       // workspace: one float
  unsigned* dbg;     // debug checks: non-finite flag, else null
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

// NVFP4 dynamic tensor scale g = RN_fp32(max |x| / 2688) of a [rows, cols]
// tensor (cols a multiple of 32) written to g_out; partials: kAmaxPartials
// floats of workspace.
hipError_t launch_nvfp4_tensor_scale(const void* x, int dtype, int64_t rows, int64_t cols,
                                     int64_t ldx, float* partials, float* g_out,
                                     unsigned* dbg, hipStream_t s);

// Weights with least-squared-error scales (MXFP4: block step; NVFP4: block,
// tensor, block).  Workspace (NVFP4): kAmaxPartials floats, then 2 * rows
// doubles (per-row sums of the tensor step), 16-byte aligned.
struct MseArgs {
  const void* x; int dtype;
  int64_t rows, cols, ldx;
  int fmt;
  uint8_t* codes; int64_t ld_codes;
  uint8_t* scales; int64_t ld_scales;
  float* tensor_scale_out;   // NVFP4
  void* ws;
  unsigned* dbg;
};
int64_t mse_workspace_bytes(int fmt, int64_t rows);

// Offline SVD split W [n][k] ~= (L1 L2)^T + R (rank-r truncated SVD by
// subspace iteration).
struct LowrankSplitArgs {
  const float* w; int64_t n, k, ldw;
  int rank, iters;
  uint16_t* l1t;      // bf16 [rank][k]
  uint16_t* l2t;      // bf16 [n][rank]
  float* resid; int64_t ld_resid;
  float* sigma;       // optional [rank]
  void* ws;
};
int64_t lowrank_split_workspace(int64_t n, int64_t k, int rank);
hipError_t launch_lowrank_split(const LowrankSplitArgs& a, hipStream_t s);
hipError_t launch_quantize_mse(const MseArgs& a, hipStream_t s);

}  // namespace mxq
