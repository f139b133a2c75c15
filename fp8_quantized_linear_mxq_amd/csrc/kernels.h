// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

struct LoraDownArgs {
  const uint16_t* x;   // bf16 [rows][ldx]
  int64_t rows, cols, ldx;
  const uint16_t* l1t; // bf16 [rank][cols]
  int rank;
  float* u;            // [rows][ld_u]
  int64_t ld_u;
};
hipError_t launch_lora_down(const LoraDownArgs& a, hipStream_t s);

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
};

constexpr int kAmaxPartials = 1024;  // NVFP4 phase-1 grid (workspace floats)

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t s);



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
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

}  // namespace mxq
