// libmxq C ABI: argument validation and route dispatch (see include/mxq.h).
//
// Every check runs on the host before anything is enqueued, so an invalid
// call returns an mxq_status without touching the device.  Valid calls are
// asynchronous on the caller's stream; the library holds no state.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "kernels.h"
#include "mxq.h"

namespace {

using namespace mxq;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int block_of(int fmt) { return fmt == MXQ_FMT_NVFP4 ? 16 : 32; }

// The quantized formats (BF16, unquantized activations, is separate).
bool known_fmt(int fmt) { return fmt >= MXQ_FMT_MXFP4 && fmt <= MXQ_FMT_INT4; }

int64_t code_bytes(int fmt, int64_t cols) {
  return fmt == MXQ_FMT_BF16 ? 2 * cols : fmt == MXQ_FMT_MXFP8 ? cols : cols / 2;
}

int64_t scale_bytes(int fmt, int64_t cols) {
  if (fmt == MXQ_FMT_BF16) return 0;
  const int64_t blocks = cols / block_of(fmt);
  return fmt == MXQ_FMT_INT4 ? blocks * 4 : blocks;
}

mxq_status from_hip(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_ERR_LAUNCH; }

// Validates a quantized operand's descriptor against its format.
mxq_status check_qtensor(const mxq_qtensor* t) {
  if (t && t->fmt == MXQ_FMT_BF16) {
    // unquantized bf16 values in `codes`; no scales
    if (t->reserved != 0 || t->rows < 0 || t->cols < 0) return MXQ_ERR_INVALID_ARG;
    if (t->rows == 0 || t->cols == 0) return MXQ_OK;
    if (!t->codes || t->ld_codes < 2 * t->cols) return MXQ_ERR_INVALID_ARG;
    if (!aligned(t->codes, 16) || t->ld_codes % 16) return MXQ_ERR_ALIGNMENT;
    return MXQ_OK;
  }
  if (!t || !known_fmt(t->fmt) || t->reserved != 0 || t->rows < 0 || t->cols < 0)
    return MXQ_ERR_INVALID_ARG;
  if (t->cols % block_of(t->fmt)) return MXQ_ERR_SHAPE;
  if (t->rows == 0 || t->cols == 0) return MXQ_OK;
  if (!t->codes || !t->scales) return MXQ_ERR_INVALID_ARG;
  if (t->fmt == MXQ_FMT_NVFP4 && !t->tensor_scale) return MXQ_ERR_INVALID_ARG;
  if (t->ld_codes < code_bytes(t->fmt, t->cols) || t->ld_scales < scale_bytes(t->fmt, t->cols))
    return MXQ_ERR_INVALID_ARG;
  if (!aligned(t->codes, 16) || t->ld_codes % 16 || !aligned(t->scales, 4) || t->ld_scales % 4)
    return MXQ_ERR_ALIGNMENT;
  if (t->fmt == MXQ_FMT_INT4 && (!aligned(t->scales, 16) || t->ld_scales % 16))
    return MXQ_ERR_ALIGNMENT;
  return MXQ_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// MXQ_DEBUG_CHECKS=1 in the environment (read at every call) turns on the
// device-side NaN / Inf checks of the quantize and format-choice kernels.
bool debug_checks() {
  const char* e = std::getenv("MXQ_DEBUG_CHECKS");
  return e && e[0] == '1' && e[1] == 0;
}

// MXQ_NVFP4_TWO_PASS=1 (read at every call) makes the dynamic NVFP4
// quantize take its two-pass kernels (an amax pass, then the quantize pass)
// even where the one-pass kernel fits; both give identical results.
bool nvfp4_two_pass() {
  const char* e = std::getenv("MXQ_NVFP4_TWO_PASS");
  return e && e[0] == '1' && e[1] == 0;
}

// Run once a call has passed validation and is about to enqueue work: a
// usable device, and in debug mode the non-finite flag a previous call may
// have set (read and cleared synchronously).  *dbg receives the flag's
// device address for the kernels (null outside debug mode).
mxq_status device_entry(unsigned** dbg) {
  *dbg = nullptr;
  int dev = -1, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0 || hipGetDevice(&dev) != hipSuccess)
    return MXQ_ERR_NO_DEVICE;
  if (!debug_checks()) return MXQ_OK;
  unsigned* flag = nullptr;
  if (nonfinite_flag_ptr(&flag) != hipSuccess) return MXQ_ERR_LAUNCH;
  unsigned v = 0;
  if (hipMemcpy(&v, flag, sizeof v, hipMemcpyDeviceToHost) != hipSuccess) return MXQ_ERR_LAUNCH;
  if (v != 0) {
    const unsigned zero = 0;
    if (hipMemcpy(flag, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
      return MXQ_ERR_LAUNCH;
    return MXQ_ERR_NONFINITE;
  }
  *dbg = flag;
  return MXQ_OK;
}

}  // namespace

extern "C" {

int32_t mxq_version(void) { return MXQ_VERSION; }

const char* mxq_status_string(int32_t status) {
  switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_INVALID_ARG: return "invalid argument";
    case MXQ_ERR_UNSUPPORTED: return "unsupported combination";
    case MXQ_ERR_ALIGNMENT: return "misaligned pointer or leading dimension";
    case MXQ_ERR_SHAPE: return "shape not a multiple of the block, tile or rotation size";
    case MXQ_ERR_WORKSPACE: return "workspace missing or too small";
    case MXQ_ERR_NO_DEVICE: return "no HIP device";
    case MXQ_ERR_LAUNCH: return "kernel launch failed";
    case MXQ_ERR_NONFINITE: return "NaN or Inf input seen by an earlier call (debug checks)";
    default: return "unknown status";
  }
}

mxq_status mxq_storage(int32_t fmt, int64_t cols, int64_t* code_b, int64_t* scale_b) {
  if (!known_fmt(fmt) || cols < 0 || !code_b || !scale_b) return MXQ_ERR_INVALID_ARG;
  if (cols % block_of(fmt)) return MXQ_ERR_SHAPE;
  *code_b = code_bytes(fmt, cols);
  *scale_b = scale_bytes(fmt, cols);
  return MXQ_OK;
}

int64_t mxq_workspace_size(int32_t op, int64_t rows, int64_t cols, int32_t fmt) {
  if (rows < 0 || cols < 0) return -1;
  switch (op) {
    case MXQ_OP_QUANTIZE:
      if (!known_fmt(fmt)) return -1;
      return fmt == MXQ_FMT_NVFP4 ? (int64_t)kAmaxPartials * 4 : 0;
    case MXQ_OP_GEMM:
      // rows = M, cols = N (weight rows), fmt = the weight format: narrow
      // INT4 weight groups split K into fp32 partials
      if (!known_fmt(fmt)) return -1;
      return fmt == MXQ_FMT_INT4 ? gemm_dq_workspace(rows, cols) : 0;
    case MXQ_OP_SELECT:
      // amax partials, the tensor scale, per-row SSE for up to 4 candidates
      return (int64_t)kAmaxPartials * 4 + 64 + rows * 4 * 8;
    case MXQ_OP_LOWRANK_SPLIT:
      // rows = N, cols = K, fmt = the rank
      if (fmt < 1 || fmt > 128 || fmt > rows || fmt > cols) return -1;
      return lowrank_split_workspace(rows, cols, fmt);
    case MXQ_OP_QUANTIZE_MSE:
      if (fmt != MXQ_FMT_MXFP4 && fmt != MXQ_FMT_NVFP4) return -1;
      return mse_workspace_bytes(fmt, rows);
    default:
      return -1;
  }
}

int32_t mxq_act_format_for_step(const uint8_t* table, int32_t n_layers, int32_t n_buckets,
                                int32_t layer, int32_t step, int32_t num_steps) {
  if (!table || n_layers <= 0 || n_buckets <= 0 || layer < 0 || layer >= n_layers ||
      num_steps <= 0 || step < 0 || step >= num_steps)
    return -1;
  int64_t bucket = ((int64_t)n_buckets * step) / num_steps;
  if (bucket > n_buckets - 1) bucket = n_buckets - 1;
  return table[(int64_t)layer * n_buckets + bucket];
}

}  // extern "C"

// mxq_quantize and its allocation-free variant: with `noalloc` the NVFP4
// amax partials go to the library's per-device scratch array instead of a
// caller workspace.
static mxq_status quantize_impl(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                int64_t ldx, int32_t hadamard_n,
                                const float* static_tensor_scale, const void* lr_l1t,
                                int32_t lr_rank, float* lr_u, int64_t ld_u, mxq_qtensor* out,
                                void* workspace, size_t ws_bytes, bool noalloc, bool packed,
                                void* stream) {
  if (!out || (dtype != MXQ_DT_F32 && dtype != MXQ_DT_BF16) || rows < 0 || cols < 0)
    return MXQ_ERR_INVALID_ARG;
  if (!known_fmt(out->fmt) || out->rows != rows || out->cols != cols) return MXQ_ERR_INVALID_ARG;
  if (hadamard_n != 0 && hadamard_n != 16 && hadamard_n != 32 && hadamard_n != 128)
    return MXQ_ERR_INVALID_ARG;
  if (lr_rank < 0 || lr_rank > 128 || lr_rank % 16) return MXQ_ERR_INVALID_ARG;
  // the kernels take 32-element runs of a row (NVFP4's 16-blocks in pairs)
  if (cols % 32 || (hadamard_n && cols % hadamard_n)) return MXQ_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MXQ_OK;
  if (rows * (cols / 8) >= (int64_t)1 << 32) return MXQ_ERR_SHAPE;
  if (!x || ldx < cols) return MXQ_ERR_INVALID_ARG;
  const int esz = dtype == MXQ_DT_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ldx * esz) % 16) return MXQ_ERR_ALIGNMENT;
  mxq_status st = check_qtensor(out);
  if (st != MXQ_OK) return st;
  if (packed && lr_rank == 0) return MXQ_ERR_INVALID_ARG;
  // the packed L1 order is read by the fused quantize + projection kernel:
  // bf16 input, no rotation, columns a multiple of 128
  if (packed && (dtype != MXQ_DT_BF16 || hadamard_n != 0)) return MXQ_ERR_UNSUPPORTED;
  if (packed && cols % 128) return MXQ_ERR_SHAPE;
  if (lr_rank > 0) {
    if (dtype != MXQ_DT_BF16) return MXQ_ERR_UNSUPPORTED;
    if (!lr_l1t || !lr_u || ld_u < lr_rank) return MXQ_ERR_INVALID_ARG;
    if (!aligned(lr_l1t, 16) || !aligned(lr_u, 16) || ld_u % 4) return MXQ_ERR_ALIGNMENT;
  }
  const bool dynamic_nv = out->fmt == MXQ_FMT_NVFP4 && !static_tensor_scale;
  if (!noalloc && dynamic_nv && (!workspace || ws_bytes < (size_t)kAmaxPartials * 4))
    return MXQ_ERR_WORKSPACE;
  unsigned* dbg = nullptr;
  st = device_entry(&dbg);
  if (st != MXQ_OK) return st;
  if (noalloc) {
    // the partials never outgrow the scratch: one per amax workgroup, at
    // most kAmaxPartials whatever the input size
    size_t bytes = 0;
    if (quantize_scratch(&workspace, &bytes) != hipSuccess) return MXQ_ERR_LAUNCH;
    if (bytes < (size_t)kAmaxPartials * 4) return MXQ_ERR_WORKSPACE;
    ws_bytes = bytes;
  }

  QuantizeArgs a;
  a.x = x;
  a.dtype = dtype;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ldx;
  a.hadamard_n = hadamard_n;
  a.fmt = out->fmt;
  a.codes = static_cast<uint8_t*>(out->codes);
  a.ld_codes = out->ld_codes;
  a.scales = static_cast<uint8_t*>(out->scales);
  a.ld_scales = out->ld_scales;
  a.tensor_scale_out = out->tensor_scale;
  a.static_tensor_scale = static_tensor_scale;
  a.partials = static_cast<float*>(workspace);
  a.dbg = dbg;
  a.nv_two_pass = nvfp4_two_pass();
  LoraDownArgs l;
  a.lr = nullptr;
  if (lr_rank > 0) {
    l.x = static_cast<const uint16_t*>(x);
    l.rows = rows;
    l.cols = cols;
    l.ldx = ldx;
    l.l1t = static_cast<const uint16_t*>(lr_l1t);
    l.rank = lr_rank;
    l.u = lr_u;
    l.ld_u = ld_u;
    l.packed = packed;
    a.lr = &l;
  }
  hipError_t e = launch_quantize(a, as_stream(stream));
  return from_hip(e);
}

extern "C" {

mxq_status mxq_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                        int32_t hadamard_n, const float* static_tensor_scale,
                        const void* lr_l1t, int32_t lr_rank, float* lr_u, int64_t ld_u,
                        mxq_qtensor* out, void* workspace, size_t ws_bytes, void* stream) {
  return quantize_impl(x, dtype, rows, cols, ldx, hadamard_n, static_tensor_scale, lr_l1t,
                       lr_rank, lr_u, ld_u, out, workspace, ws_bytes, false, false, stream);
}

mxq_status mxq_quantize_lrp(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                            int32_t hadamard_n, const float* static_tensor_scale,
                            const void* lr_l1p, int32_t lr_rank, float* lr_u, int64_t ld_u,
                            mxq_qtensor* out, void* workspace, size_t ws_bytes, void* stream) {
  return quantize_impl(x, dtype, rows, cols, ldx, hadamard_n, static_tensor_scale, lr_l1p,
                       lr_rank, lr_u, ld_u, out, workspace, ws_bytes, false, true, stream);
}

mxq_status mxq_pack_l1t(const void* l1t, int32_t rank, int64_t cols, void* l1p, void* stream) {
  if (rank < 16 || rank > 128 || rank % 16 || cols < 0) return MXQ_ERR_INVALID_ARG;
  if (cols % 128) return MXQ_ERR_SHAPE;
  if (cols == 0) return MXQ_OK;
  if (!l1t || !l1p) return MXQ_ERR_INVALID_ARG;
  if (!aligned(l1t, 16) || !aligned(l1p, 16)) return MXQ_ERR_ALIGNMENT;
  unsigned* dbg = nullptr;
  const mxq_status st = device_entry(&dbg);
  if (st != MXQ_OK) return st;
  return from_hip(launch_pack_l1t(static_cast<const uint16_t*>(l1t), rank, cols,
                                  static_cast<uint16_t*>(l1p), as_stream(stream)));
}

mxq_status mxq_quantize_noalloc(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                int64_t ldx, int32_t hadamard_n,
                                const float* static_tensor_scale, const void* lr_l1t,
                                int32_t lr_rank, float* lr_u, int64_t ld_u, mxq_qtensor* out,
                                void* stream) {
  return quantize_impl(x, dtype, rows, cols, ldx, hadamard_n, static_tensor_scale, lr_l1t,
                       lr_rank, lr_u, ld_u, out, nullptr, 0, true, false, stream);
}

static mxq_status gemm_checks(const mxq_qtensor* a, const mxq_qtensor* w, const float* lr_u,
                              int64_t ld_u, const void* lr_l2t, int32_t lr_rank, void* out,
                              int64_t ld_out, int64_t n_out) {
  mxq_status st = check_qtensor(a);
  if (st != MXQ_OK) return st;
  st = check_qtensor(w);
  if (st != MXQ_OK) return st;
  if (a->cols != w->cols) return MXQ_ERR_SHAPE;
  if (n_out < 0 || lr_rank < 0 || lr_rank > 128 || lr_rank % 16) return MXQ_ERR_INVALID_ARG;
  // activations: MXFP4, MXFP8, NVFP4 or bf16; weights: MXFP4, NVFP4 or INT4
  if (a->fmt == MXQ_FMT_INT4 || w->fmt == MXQ_FMT_MXFP8 || w->fmt == MXQ_FMT_BF16)
    return MXQ_ERR_UNSUPPORTED;
  if (a->rows == 0 || w->rows == 0 || n_out == 0) return MXQ_OK;
  if (a->cols % 128) return MXQ_ERR_SHAPE;
  if (a->rows > INT32_MAX || w->rows > INT32_MAX || a->cols > INT32_MAX || n_out > INT32_MAX)
    return MXQ_ERR_SHAPE;
  if (!out || ld_out < n_out) return MXQ_ERR_INVALID_ARG;
  if (!aligned(out, 2)) return MXQ_ERR_ALIGNMENT;
  if (lr_rank > 0) {
    if (!lr_u || !lr_l2t || ld_u < lr_rank) return MXQ_ERR_INVALID_ARG;
    if (!aligned(lr_u, 16) || ld_u % 4 || !aligned(lr_l2t, 16)) return MXQ_ERR_ALIGNMENT;
  }
  return MXQ_OK;
}

// One GEMM launch of the route for (a->fmt, w->fmt).  With cv_c > 0 the
// activation operand is the implicit im2col of a 3x3 convolution over an
// [images * cv_h * cv_w][cv_c] pixel-row input (K = w->cols = 9 * cv_c).
static hipError_t gemm_launch(const mxq_qtensor* a, const mxq_qtensor* w, const int32_t* col_map,
                              const float* lr_u, int64_t ld_u, const void* lr_l2t,
                              int32_t lr_rank, const void* bias, void* out, int64_t ld_out,
                              int64_t n_out, void* workspace, size_t ws_bytes, hipStream_t s,
                              int64_t cv_h = 0, int64_t cv_w = 0, int64_t cv_c = 0) {
  GemmArgs g;
  g.cv_h = cv_h;
  g.cv_w = cv_w;
  g.cv_c = cv_c;
  g.ws = static_cast<float*>(workspace);
  g.ws_bytes = workspace ? (int64_t)ws_bytes : 0;
  g.a_fmt = a->fmt;
  g.w_fmt = w->fmt;
  g.a_codes = static_cast<const uint8_t*>(a->codes);
  g.lda = a->ld_codes;
  g.a_scales = static_cast<const uint8_t*>(a->scales);
  g.ld_as = a->ld_scales;
  g.a_g = a->tensor_scale;
  g.w_codes = static_cast<const uint8_t*>(w->codes);
  g.ldw = w->ld_codes;
  g.w_scales = static_cast<const uint8_t*>(w->scales);
  g.ld_ws = w->ld_scales;
  g.w_g = w->tensor_scale;
  g.M = a->rows;
  g.N = w->rows;
  g.K = w->cols;
  g.col_map = col_map;
  g.u = lr_u;
  g.ld_u = ld_u;
  g.l2t = static_cast<const uint16_t*>(lr_l2t);
  g.rank = lr_rank;
  g.bias = static_cast<const uint16_t*>(bias);
  g.out = static_cast<uint16_t*>(out);
  g.ld_out = ld_out;
  g.n_out = n_out;
  // E2M1 x E2M1 is exact on the scaled MFMA; every other pair is dequantized
  // exactly to 16-bit operands (E4M3 MFMA products are not summed to fp32
  // accuracy on this hardware)
  if (a->fmt == MXQ_FMT_MXFP4 && w->fmt == MXQ_FMT_MXFP4) return launch_gemm_mx(g, s);
  if (w->fmt == MXQ_FMT_INT4) return launch_gemm_dq(g, s);
  return launch_gemm_dqp(g, s);
}

mxq_status mxq_gemm(const mxq_qtensor* a, const mxq_qtensor* w, const int32_t* w_out_col,
                    const float* lr_u, int64_t ld_u, const void* lr_l2t, int32_t lr_rank,
                    const void* bias, void* out, int64_t ld_out, int64_t n_out,
                    void* workspace, size_t ws_bytes, void* stream) {
  mxq_status st = gemm_checks(a, w, lr_u, ld_u, lr_l2t, lr_rank, out, ld_out, n_out);
  if (st != MXQ_OK) return st;
  if (workspace && !aligned(workspace, 16)) return MXQ_ERR_ALIGNMENT;
  if (a->rows == 0 || w->rows == 0 || n_out == 0) return MXQ_OK;
  if (!w_out_col && w->rows > n_out) return MXQ_ERR_SHAPE;
  unsigned* dbg = nullptr;
  st = device_entry(&dbg);
  if (st != MXQ_OK) return st;
  return from_hip(gemm_launch(a, w, w_out_col, lr_u, ld_u, lr_l2t, lr_rank, bias, out, ld_out,
                              n_out, workspace, ws_bytes, as_stream(stream)));
}

mxq_status mxq_gemm_mixed(const mxq_qtensor* a, const mxq_qtensor* w_groups, int32_t n_groups,
                          const int32_t* w_perm, const float* lr_u, int64_t ld_u,
                          const void* lr_l2t, int32_t lr_rank, const void* bias, void* out,
                          int64_t ld_out, int64_t n_out, void* workspace, size_t ws_bytes,
                          void* stream) {
  if (!w_groups || n_groups <= 0 || n_groups > 8) return MXQ_ERR_INVALID_ARG;
  if (workspace && !aligned(workspace, 16)) return MXQ_ERR_ALIGNMENT;
  int64_t total = 0;
  for (int g = 0; g < n_groups; ++g) {
    mxq_status st = gemm_checks(a, &w_groups[g], lr_u, ld_u, lr_l2t, lr_rank, out, ld_out, n_out);
    if (st != MXQ_OK) return st;
    total += w_groups[g].rows;
  }
  if (total > 0 && !w_perm) return MXQ_ERR_INVALID_ARG;
  if (a->rows == 0 || n_out == 0) return MXQ_OK;
  unsigned* dbg = nullptr;
  const mxq_status dst = device_entry(&dbg);
  if (dst != MXQ_OK) return dst;
  int64_t off = 0;
  for (int g = 0; g < n_groups; ++g) {
    const mxq_qtensor* w = &w_groups[g];
    if (w->rows > 0) {
      hipError_t e = gemm_launch(a, w, w_perm + off, lr_u, ld_u, lr_l2t, lr_rank, bias, out,
                                 ld_out, n_out, workspace, ws_bytes, as_stream(stream));
      if (e != hipSuccess) return MXQ_ERR_LAUNCH;
    }
    off += w->rows;
  }
  return MXQ_OK;
}

mxq_status mxq_conv3x3_gemm_mixed(const mxq_qtensor* x, int64_t height, int64_t width,
                                  const mxq_qtensor* w_groups, int32_t n_groups,
                                  const int32_t* w_perm, const void* bias, void* out,
                                  int64_t ld_out, int64_t n_out, void* workspace,
                                  size_t ws_bytes, void* stream) {
  if (!w_groups || n_groups <= 0 || n_groups > 8) return MXQ_ERR_INVALID_ARG;
  mxq_status st = check_qtensor(x);
  if (st != MXQ_OK) return st;
  if (height <= 0 || width <= 0 || n_out < 0) return MXQ_ERR_INVALID_ARG;
  if (x->fmt == MXQ_FMT_INT4 || x->fmt == MXQ_FMT_BF16) return MXQ_ERR_UNSUPPORTED;
  if (workspace && !aligned(workspace, 16)) return MXQ_ERR_ALIGNMENT;
  if (height > INT32_MAX / width) return MXQ_ERR_SHAPE;
  const int64_t C = x->cols, hw = height * width;
  // a K-tile (128) never spans two taps; pixels are whole images; the
  // kernels' tap lookup is exact up to 2**20 channels
  if (C % 128 || x->rows % hw || C > (1 << 20)) return MXQ_ERR_SHAPE;
  if (x->rows > INT32_MAX || 9 * C > INT32_MAX || n_out > INT32_MAX) return MXQ_ERR_SHAPE;
  int64_t total = 0;
  for (int g = 0; g < n_groups; ++g) {
    const mxq_qtensor* w = &w_groups[g];
    st = check_qtensor(w);
    if (st != MXQ_OK) return st;
    if (w->fmt == MXQ_FMT_MXFP8 || w->fmt == MXQ_FMT_BF16) return MXQ_ERR_UNSUPPORTED;
    // the scaled-MFMA route (MXFP4 x MXFP4) reads no implicit im2col
    if (x->fmt == MXQ_FMT_MXFP4 && w->fmt == MXQ_FMT_MXFP4 && w->rows > 0)
      return MXQ_ERR_UNSUPPORTED;
    if (w->cols != 9 * C) return MXQ_ERR_SHAPE;
    if (w->rows > INT32_MAX) return MXQ_ERR_SHAPE;
    total += w->rows;
  }
  if (x->rows == 0 || n_out == 0 || total == 0) return MXQ_OK;
  if (!out || ld_out < n_out) return MXQ_ERR_INVALID_ARG;
  if (!aligned(out, 2)) return MXQ_ERR_ALIGNMENT;
  // without a permutation a single group's row j is output column j
  if (!w_perm && (n_groups > 1 || total > n_out)) return MXQ_ERR_INVALID_ARG;
  unsigned* dbg = nullptr;
  st = device_entry(&dbg);
  if (st != MXQ_OK) return st;
  int64_t off = 0;
  for (int g = 0; g < n_groups; ++g) {
    const mxq_qtensor* w = &w_groups[g];
    if (w->rows > 0) {
      hipError_t e = gemm_launch(x, w, w_perm ? w_perm + off : nullptr, nullptr, 0, nullptr, 0,
                                 bias, out, ld_out, n_out, workspace, ws_bytes,
                                 as_stream(stream), height, width, C);
      if (e != hipSuccess) return MXQ_ERR_LAUNCH;
    }
    off += w->rows;
  }
  return MXQ_OK;
}

mxq_status mxq_quantize_mse(const void* w, int32_t dtype, int64_t rows, int64_t cols,
                            int64_t ldw, mxq_qtensor* out, void* workspace, size_t ws_bytes,
                            void* stream) {
  if (!out || (dtype != MXQ_DT_F32 && dtype != MXQ_DT_BF16) || rows < 0 || cols < 0)
    return MXQ_ERR_INVALID_ARG;
  if (out->fmt != MXQ_FMT_MXFP4 && out->fmt != MXQ_FMT_NVFP4)
    return known_fmt(out->fmt) ? MXQ_ERR_UNSUPPORTED : MXQ_ERR_INVALID_ARG;
  if (out->rows != rows || out->cols != cols) return MXQ_ERR_INVALID_ARG;
  if (cols % 32) return MXQ_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MXQ_OK;
  if (rows * (cols / 8) >= (int64_t)1 << 32) return MXQ_ERR_SHAPE;
  if (!w || ldw < cols) return MXQ_ERR_INVALID_ARG;
  const int esz = dtype == MXQ_DT_F32 ? 4 : 2;
  if (!aligned(w, 16) || (ldw * esz) % 16) return MXQ_ERR_ALIGNMENT;
  mxq_status st = check_qtensor(out);
  if (st != MXQ_OK) return st;
  const int64_t need = mse_workspace_bytes(out->fmt, rows);
  if (need > 0 && (!workspace || ws_bytes < (size_t)need || !aligned(workspace, 16)))
    return MXQ_ERR_WORKSPACE;
  unsigned* dbg = nullptr;
  st = device_entry(&dbg);
  if (st != MXQ_OK) return st;
  MseArgs a;
  a.x = w;
  a.dtype = dtype;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ldw;
  a.fmt = out->fmt;
  a.codes = static_cast<uint8_t*>(out->codes);
  a.ld_codes = out->ld_codes;
  a.scales = static_cast<uint8_t*>(out->scales);
  a.ld_scales = out->ld_scales;
  a.tensor_scale_out = out->tensor_scale;
  a.ws = workspace;
  a.dbg = dbg;
  return from_hip(launch_quantize_mse(a, as_stream(stream)));
}

mxq_status mxq_lowrank_split(const float* w, int64_t n, int64_t k, int64_t ldw, int32_t rank,
                             int32_t iters, void* l1t, void* l2t, float* resid, int64_t ld_resid,
                             float* sigma, void* workspace, size_t ws_bytes, void* stream) {
  if (n < 0 || k < 0 || rank < 1 || rank > 128 || iters < 0 || iters > 64)
    return MXQ_ERR_INVALID_ARG;
  if (rank > n || rank > k) return MXQ_ERR_SHAPE;
  if (!w || !l1t || !l2t || !resid || ldw < k || ld_resid < k) return MXQ_ERR_INVALID_ARG;
  if (!aligned(w, 4) || !aligned(l1t, 2) || !aligned(l2t, 2) || !aligned(resid, 4) ||
      (sigma && !aligned(sigma, 4)))
    return MXQ_ERR_ALIGNMENT;
  const int64_t need = lowrank_split_workspace(n, k, rank);
  if (!workspace || ws_bytes < (size_t)need || !aligned(workspace, 256)) return MXQ_ERR_WORKSPACE;
  unsigned* dbg = nullptr;
  const mxq_status st = device_entry(&dbg);
  if (st != MXQ_OK) return st;
  LowrankSplitArgs a;
  a.w = w;
  a.n = n;
  a.k = k;
  a.ldw = ldw;
  a.rank = rank;
  a.iters = iters == 0 ? 8 : iters;
  a.l1t = static_cast<uint16_t*>(l1t);
  a.l2t = static_cast<uint16_t*>(l2t);
  a.resid = resid;
  a.ld_resid = ld_resid;
  a.sigma = sigma;
  a.ws = workspace;
  return from_hip(launch_lowrank_split(a, as_stream(stream)));
}

mxq_status mxq_select_format(const void* w, int32_t dtype, int64_t n, int64_t k, int64_t ldw,
                             const int32_t* candidates, int32_t n_cand, uint8_t* choice_out,
                             double* sse_out, int32_t* perm_out, int32_t* counts_out,
                             float* g_out, void* workspace, size_t ws_bytes, void* stream) {
  if ((dtype != MXQ_DT_F32 && dtype != MXQ_DT_BF16) || n < 0 || k < 0) return MXQ_ERR_INVALID_ARG;
  if (!candidates || n_cand <= 0 || n_cand > 4) return MXQ_ERR_INVALID_ARG;
  for (int i = 0; i < n_cand; ++i)
    if (candidates[i] != MXQ_FMT_MXFP4 && candidates[i] != MXQ_FMT_NVFP4 &&
        candidates[i] != MXQ_FMT_INT4)
      return MXQ_ERR_UNSUPPORTED;
  if (k % 32) return MXQ_ERR_SHAPE;
  if (n == 0 || k == 0) return MXQ_OK;
  if (n > INT32_MAX || n * (k / 8) >= (int64_t)1 << 32) return MXQ_ERR_SHAPE;
  if (!w || !choice_out || ldw < k) return MXQ_ERR_INVALID_ARG;
  const int esz = dtype == MXQ_DT_F32 ? 4 : 2;
  if (!aligned(w, 16) || (ldw * esz) % 16) return MXQ_ERR_ALIGNMENT;
  const int64_t need = mxq_workspace_size(MXQ_OP_SELECT, n, k, 0);
  if (!workspace || ws_bytes < (size_t)need || !aligned(workspace, 16)) return MXQ_ERR_WORKSPACE;
  unsigned* dbg = nullptr;
  const mxq_status dst = device_entry(&dbg);
  if (dst != MXQ_OK) return dst;
  SelectArgs a;
  a.dbg = dbg;
  a.w = w;
  a.dtype = dtype;
  a.n = n;
  a.k = k;
  a.ldw = ldw;
  for (int i = 0; i < 4; ++i) a.cand[i] = i < n_cand ? candidates[i] : 0;
  a.n_cand = n_cand;
  a.choice = choice_out;
  a.sse = sse_out;
  a.perm = perm_out;
  a.counts = counts_out;
  a.g_out = g_out;
  char* ws = static_cast<char*>(workspace);
  a.partials = reinterpret_cast<float*>(ws);
  a.g_ws = reinterpret_cast<float*>(ws + (size_t)kAmaxPartials * 4);
  a.sse_ws = reinterpret_cast<double*>(ws + (size_t)kAmaxPartials * 4 + 64);
  return from_hip(launch_select(a, as_stream(stream)));
}

}  // extern "C"
