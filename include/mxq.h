/*
 * mxq.h -- C ABI of libmxq: block-scaled (microscaling) quantized linear
 * layers on AMD Instinct MI355X (gfx950).
 *
 * The library computes one path:
 *   activations x [M, K] (fp32 or bf16)
 *     -> optional block-diagonal Hadamard rotation along K       (mxq_quantize)
 *     -> block quantization to MXFP4 / MXFP8 / NVFP4 (or INT4)   (mxq_quantize)
 *     -> block-scaled GEMM against pre-quantized 4-bit weights,
 *        fp32 accumulation, optional rank-r bf16 branch, bf16 out (mxq_gemm)
 *   plus the weight-side per-output-channel format choice        (mxq_select_format)
 *   and the timestep-bucket activation-format lookup             (mxq_act_format_for_step)
 *
 * Sources (pages the method is described on, cited by title and section):
 *  - "Bridging the Gap Between Promise and Performance for Microscaling FP4
 *    Quantization" (summary page): MXFP4 uses power-of-two block scales,
 *    NVFP4 small groups with block and tensor scales (the two reasons FP4
 *    fails); activations are rotated at inference by block-diagonal
 *    Hadamard rotations (modification 3).
 *  - Nunchaku / SVDQuant article, "main explanation": 4-bit weights and
 *    activations (W4A4) plus a 16-bit low-rank branch.
 *  - Chameleon format-selection article, "the format is chosen by the value
 *    distribution": per-output-channel weight format by least reconstruction
 *    error, activation format read from a table per timestep interval (ten
 *    intervals), MXFP8 forced for concatenated-feature convolutions; "hardware
 *    support" paragraph: channel-mixed formats need a grouped GEMM.
 *
 * Formats (OCP microscaling / OCP FP8 / NVFP4 definitions; the pages give no
 * bit layouts):
 *   MXFP4  E2M1 elements, one E8M0 scale per 32 elements along K
 *   MXFP8  E4M3 elements, one E8M0 scale per 32
 *   NVFP4  E2M1 elements, one E4M3 scale per 16, one fp32 tensor scale g
 *   INT4   symmetric two's-complement int4, one fp32 scale per 32 (weights)
 * Rounding: nearest, ties to even, saturating at the largest finite value,
 * decided on the exact real quotient.  Scale rules:
 *   MX     e = clamp(floor(log2 amax) - emax_elem, -127, 127), code e + 127,
 *          emax_elem = 2 (E2M1) or 8 (E4M3); amax = 0 gives code 0.
 *   NVFP4  g = RN_fp32(A / 2688), A = tensor amax; s = RN_E4M3(amax / (6 g)).
 *   INT4   s = RN_fp32(amax / 7); q = clamp(RNE(x / s), -7, 7).
 *
 * Storage (all device memory, row-major, K contiguous):
 *   codes   4-bit formats: [rows][K/2] bytes, element 2i in the low nibble
 *           of byte i; MXFP8: [rows][K] bytes.
 *   scales  MX: [rows][K/32] E8M0 bytes; NVFP4: [rows][K/16] E4M3 bytes;
 *           INT4: [rows][K/32] fp32.
 *   tensor_scale  NVFP4 only: one fp32 in device memory.
 * Weights, like nn.Linear, are stored [out][in] with the reduction index
 * contiguous: W [N][K], the low-rank factors as L1^T [r][K] and L2^T [N][r].
 *
 * Conventions for every entry point:
 *  - Ownership: the caller allocates and owns every buffer (inputs, outputs,
 *    workspace).  The library never allocates, frees or synchronizes.
 *  - Streams: work is enqueued on `stream` (a hipStream_t passed as void*;
 *    NULL is the default stream) and the call returns without waiting.
 *  - Errors: invalid arguments are reported synchronously, before any work
 *    is enqueued, as an mxq_status; a call that would enqueue work returns
 *    MXQ_ERR_NO_DEVICE when no HIP device is available (checked after the
 *    arguments); a failed launch returns MXQ_ERR_LAUNCH.  Faults inside
 *    kernels surface at the caller's next synchronization.  No C++
 *    exception crosses this interface.
 *  - NaN or Inf inputs are outside the contract: results are unspecified
 *    (every code and scale written stays a valid bit pattern and no memory
 *    outside the outputs is touched).  With MXQ_DEBUG_CHECKS=1 in the
 *    environment (read at every call), mxq_quantize and mxq_select_format
 *    flag such inputs on the device, and the next call that enqueues work
 *    on that device returns MXQ_ERR_NONFINITE (and clears the flag) instead
 *    of running.  Debug mode reads the flag synchronously at every such
 *    call, so it synchronizes the device and cannot be graph-captured.
 *  - Apart from that debug flag, mxq_quantize_noalloc's scratch array and
 *    the barrier slots of the one-pass NVFP4 quantize (a ring of 16 per
 *    device, about 25 KB each, zero at load and left zero by every call) the
 *    library keeps no state; calls on distinct streams are independent,
 *    except mxq_quantize_noalloc calls that overlap in time on one device
 *    (they share its scratch array) and dynamic NVFP4 quantizes: one whose
 *    grid cannot be resident at once within about a second, because other
 *    work holds the compute units, writes a NaN tensor scale.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_VERSION 1

typedef enum mxq_status {
  MXQ_OK = 0,
  MXQ_ERR_INVALID_ARG = 1, /* null pointer, negative size, unknown enum      */
  MXQ_ERR_UNSUPPORTED = 2, /* valid but unimplemented combination            */
  MXQ_ERR_ALIGNMENT = 3,   /* pointer or leading dimension misaligned        */
  MXQ_ERR_SHAPE = 4,       /* K not a multiple of the block / tile / rotation*/
  MXQ_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required     */
  MXQ_ERR_NO_DEVICE = 6,   /* no HIP device available                        */
  MXQ_ERR_LAUNCH = 7,      /* kernel launch failed                           */
  MXQ_ERR_NONFINITE = 8    /* debug checks: an earlier call saw NaN / Inf    */
} mxq_status;

typedef enum mxq_format {
  MXQ_FMT_MXFP4 = 1,
  MXQ_FMT_MXFP8 = 2,
  MXQ_FMT_NVFP4 = 3,
  MXQ_FMT_INT4 = 4,
  /* Unquantized bf16 activations (4-bit weights, 16-bit activations; the
   * Nunchaku article, "kernels and supported hardware": the second kernel
   * type, for the adaptive-normalization layers that need the precision).
   * Only as mxq_gemm / mxq_gemm_mixed's `a`: codes holds the bf16 values
   * [rows][ld_codes bytes] (16-byte aligned, ld_codes a multiple of 16),
   * scales and tensor_scale are unused.  Not a quantize target. */
  MXQ_FMT_BF16 = 5
} mxq_format;

typedef enum mxq_dtype { MXQ_DT_F32 = 1, MXQ_DT_BF16 = 2 } mxq_dtype;

/* A quantized [rows, cols] tensor (cols = K, the reduction axis). */
typedef struct mxq_qtensor {
  int32_t fmt;           /* mxq_format                                      */
  int32_t reserved;      /* must be 0                                       */
  int64_t rows;
  int64_t cols;
  void* codes;           /* device; 16-byte aligned                         */
  int64_t ld_codes;      /* bytes between rows; multiple of 16              */
  void* scales;          /* device; 4-byte aligned                          */
  int64_t ld_scales;     /* bytes between rows; multiple of 4               */
  float* tensor_scale;   /* NVFP4: device pointer to g; otherwise NULL      */
} mxq_qtensor;

/*
 * mxq_quantize -- rotate (optional) and block-quantize a [rows, cols] tensor.
 *
 * Computes the scale and element rules above (Microscaling FP4 summary, the
 * two reasons FP4 fails) on r = x, or on r = x H_bd when hadamard_n > 0
 * (same summary, modification 3): H_bd is block-diagonal along K with
 * n-point Sylvester blocks scaled by 1/sqrt(n); the block sums are exact and
 * r = RN_fp32(RN_fp64(c_n * S)) with c_n the float64 nearest 1/sqrt(n).
 * The sums are exact when each n-block's inputs span at most 53 - log2(n) - 1
 * bits between the top bit of the largest and the last mantissa bit of the
 * smallest nonzero element (always true for bf16 inputs within 2**38).
 *
 *  x           device, dtype elements, row stride ldx (elements, >= cols);
 *              16-byte aligned, ldx * sizeof(dtype) a multiple of 16.
 *  dtype       MXQ_DT_F32 or MXQ_DT_BF16.
 *  hadamard_n  0 (none), 16, 32 or 128; must divide cols.
 *  static_tensor_scale  NVFP4 only: device pointer to a caller-chosen g
 *              (then block scales saturate at 448), or NULL for the dynamic
 *              g computed from this tensor: one pass over x when its blocks
 *              fit in the registers of one resident grid (up to about 16M
 *              elements, 2048 workgroups; the workgroups meet in a
 *              device-wide maximum), else two passes (an amax pass, then the
 *              quantize).  MXQ_NVFP4_TWO_PASS=1 in the environment (read at
 *              every call) forces the two passes; the results are identical.
 *  lr_l1t, lr_rank, lr_u, ld_u  optional fused low-rank down projection of
 *              the SVDQuant branch (Nunchaku article, main explanation):
 *              u = x L1 on the unrotated bf16 input, with L1^T [lr_rank][cols]
 *              bf16 (row stride cols) and u [rows][ld_u] fp32 out.
 *              lr_rank is 0 (off) or a multiple of 16 up to 128; bf16 x only.
 *  out         out->fmt, codes, scales, ld_* and (NVFP4) tensor_scale set by
 *              the caller; rows/cols must equal rows/cols.  For NVFP4 the
 *              tensor scale used is written to *out->tensor_scale.
 *  workspace   device scratch of mxq_workspace_size(MXQ_OP_QUANTIZE, ...)
 *              bytes (only dynamic NVFP4 needs any).
 * Returns MXQ_ERR_SHAPE when cols is not a multiple of 32 (for NVFP4 too:
 * its 16-blocks are quantized in pairs) or of hadamard_n.  rows == 0 or
 * cols == 0 is a no-op: MXQ_OK once the checks that need no data have passed
 * (dtype, out's format and sizes, hadamard_n, lr_rank's range, the column
 * multiples); pointers, alignment, the workspace and the conditions of the
 * low-rank path are checked for non-empty inputs only.
 */
mxq_status mxq_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                        int64_t ldx, int32_t hadamard_n,
                        const float* static_tensor_scale,
                        const void* lr_l1t, int32_t lr_rank, float* lr_u, int64_t ld_u,
                        mxq_qtensor* out, void* workspace, size_t ws_bytes,
                        void* stream);

/*
 * mxq_pack_l1t -- rearrange the first low-rank factor L1^T [rank][cols]
 * (bf16, row stride cols, K contiguous) into the order in which the fused
 * quantize + low-rank kernel reads it (Nunchaku article, main explanation:
 * L1 is part of the weight, prepared once).  Same size, rank * cols bf16:
 * 16-byte piece i = ((g * rank/16 + t) * 4 + j) * 64 + l holds
 * L1^T[16 t + l % 16][128 g + 32 (l / 16) + 8 j + (0 .. 7)], so one wave's
 * load of a fragment set is one contiguous kilobyte.  l1t and l1p are device
 * pointers, 16-byte aligned, not overlapping; rank a multiple of 16 in
 * [16, 128]; cols a multiple of 128 (else MXQ_ERR_SHAPE).  Enqueued on stream.
 */
mxq_status mxq_pack_l1t(const void* l1t, int32_t rank, int64_t cols, void* l1p, void* stream);

/*
 * mxq_quantize_lrp -- mxq_quantize with the low-rank factor given in the
 * packed order of mxq_pack_l1t (lr_l1p) instead of L1^T rows.  Same results
 * (codes, scales, tensor scale and u bit-identical to mxq_quantize with the
 * unpacked L1^T); the projection's factor reads are whole contiguous
 * kilobytes.  It takes the fused quantize + projection path only: lr_rank a
 * multiple of 16 in [16, 128] (0 is MXQ_ERR_INVALID_ARG), bf16 x and
 * hadamard_n 0 (else MXQ_ERR_UNSUPPORTED), cols a multiple of 128 (else
 * MXQ_ERR_SHAPE); like the other low-rank conditions these are checked for
 * non-empty inputs.  Other arguments, workspace and errors as mxq_quantize.
 */
mxq_status mxq_quantize_lrp(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                            int64_t ldx, int32_t hadamard_n,
                            const float* static_tensor_scale,
                            const void* lr_l1p, int32_t lr_rank, float* lr_u, int64_t ld_u,
                            mxq_qtensor* out, void* workspace, size_t ws_bytes,
                            void* stream);

/*
 * mxq_quantize_noalloc -- mxq_quantize with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * results and errors as mxq_quantize.  The dynamic NVFP4 tensor scale in
 * its one-pass form uses the library's barrier slots, as mxq_quantize does;
 * in its two-pass form the scratch it needs (its amax partials, at most 1024
 * floats whatever the input size, so no input is too large for it) lives in
 * a 4 KB array of the library's own, one per device, held until the process
 * ends.  The library looks up the address of each such array on the first
 * call on each device (that call must run with the device current); nothing
 * is allocated or freed, here or later.  Calls on one device share the array: calls that overlap in time on
 * one device (different streams, no ordering between them) race and may
 * produce wrong NVFP4 tensor scales; calls ordered on one stream do not.
 */
mxq_status mxq_quantize_noalloc(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                int64_t ldx, int32_t hadamard_n,
                                const float* static_tensor_scale,
                                const void* lr_l1t, int32_t lr_rank, float* lr_u, int64_t ld_u,
                                mxq_qtensor* out, void* stream);

/*
 * mxq_gemm -- y = RN_bf16(alpha * Q(a) Q(w)^T + u L2 + bias) for one weight
 * format (Nunchaku article, main explanation: 4-bit GEMM plus the 16-bit
 * low-rank branch added in the same output).
 *
 *  a           quantized activations [M, K]: MXFP4, MXFP8 or NVFP4; or
 *              unquantized bf16 activations (MXQ_FMT_BF16), taken exactly.
 *  w           quantized weights [N, K]: MXFP4, NVFP4 or INT4.  Every pair
 *              is supported: MXFP4 x MXFP4 on the scaled MFMA; the others
 *              dequantize exactly to fp16 (NVFP4 x NVFP4) or bf16 operands;
 *              INT4 rows sum each 32-block and apply its fp32 scale.
 *              Input domain of the dequantizing routes (every pair except
 *              MXFP4 x MXFP4): an MX operand's values are formed with its
 *              exponent raised by 10 (MXFP8) or 2 (MXFP4), undone exactly
 *              in the epilogue, so every E8M0 code down to 0 (2**-127)
 *              dequantizes exactly; in exchange MXFP8 blocks must have scale
 *              codes <= 236 (block amax below 2**117) and MXFP4 blocks codes
 *              <= 250 (amax below 2**126).
 * Error bound: |y - y_exact| <= 1e-5 (1 + 2**-8) S + 2**-8 |y_exact| + 2**-133
 * with S = alpha sum_k |a w| + sum_j |u_j L2_jn| (the last two terms are the
 * bf16 output rounding, 2**-133 covering subnormal outputs).
 *  alpha       the product of the NVFP4 tensor scales of a and w that are
 *              NVFP4 (read from their tensor_scale pointers on the device).
 *  w_out_col   optional device int32[N]: weight row n writes output column
 *              w_out_col[n] (the grouped mixed-format layout); NULL = n.
 *              Entries outside [0, n_out) are skipped.
 *  lr_u, ld_u, lr_l2t, lr_rank  optional low-rank branch: u [M][ld_u] fp32
 *              from mxq_quantize, L2^T [n_out][lr_rank] bf16 indexed by the
 *              output column; lr_rank 0 = off, else a multiple of 16 <= 128.
 *  bias        optional device bf16 [n_out], indexed by output column.
 *  out         device bf16 [M][ld_out], n_out columns; 4-byte aligned.
 *  workspace   optional (NULL, or 16-byte aligned device memory of ws_bytes):
 *              INT4 weights too narrow to fill the GPU (at most 128 output
 *              tiles of 128 x 128) split K into fp32 partial sums there (up
 *              to 16 splits of M * N floats; mxq_workspace_size(MXQ_OP_GEMM,
 *              M, N, w->fmt) bytes cover every K, and a smaller workspace
 *              takes as many splits as fit), which a second kernel adds in a
 *              fixed order (results are deterministic for a given workspace
 *              size; they may differ from the unsplit sum by fp32 rounding,
 *              within the same error bound).  Otherwise, and for every other
 *              route and with a low-rank branch, it is unused.
 * Requirements: a->cols == w->cols == K, K a multiple of 128.
 * M or N of 0 is a no-op.  Accumulation is fp32; long K is summed in slabs.
 */
mxq_status mxq_gemm(const mxq_qtensor* a, const mxq_qtensor* w, const int32_t* w_out_col,
                    const float* lr_u, int64_t ld_u, const void* lr_l2t, int32_t lr_rank,
                    const void* bias, void* out, int64_t ld_out, int64_t n_out,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * mxq_gemm_mixed -- the grouped GEMM for per-output-channel weight formats
 * (Chameleon article, "hardware support" paragraph: mixed formats split the
 * product into groups).  w_groups[g] holds the rows of format group g, in
 * order; w_perm (device int32, sum of group rows) gives each grouped row's
 * output column, group after group.  Each group runs mxq_gemm's route for
 * its format on the same stream; the low-rank branch and bias, if given,
 * are added exactly once per output column.  The workspace is mxq_gemm's,
 * shared by the groups in turn (size it for the largest INT4 group).
 */
mxq_status mxq_gemm_mixed(const mxq_qtensor* a, const mxq_qtensor* w_groups, int32_t n_groups,
                          const int32_t* w_perm,
                          const float* lr_u, int64_t ld_u, const void* lr_l2t, int32_t lr_rank,
                          const void* bias, void* out, int64_t ld_out, int64_t n_out,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * mxq_conv3x3_gemm_mixed -- a 3x3, stride-1, zero-padding-1 convolution as the
 * grouped mixed-format GEMM of mxq_gemm_mixed, with the activation operand
 * read as the implicit im2col of the quantized input (Chameleon article,
 * "routing" paragraph: the concatenated-feature convolutions, kept at MXFP8).
 * No im2col matrix is built or quantized: each 32- or 16-block of an im2col
 * row is either a block of one input pixel's channel row, which quantizes to
 * the same codes and scale in the input, or lies wholly in the zero padding
 * and adds nothing (and the NVFP4 tensor amax is the input's, since every
 * pixel is some output's centre tap).
 *
 *  x           quantized input [images * height * width][C] (pixel rows in
 *              row-major image, y, x order; C channels): MXFP8, NVFP4 or
 *              MXFP4 (not bf16).  C must be a multiple of 128, at most 2**20.
 *  height, width  the spatial size of each image (> 0); x->rows must be a
 *              multiple of height * width.
 *  w_groups, n_groups, w_perm  weight groups as in mxq_gemm_mixed, each
 *              [rows][9 * C] with K index (ky * 3 + kx) * C + c for tap
 *              (ky, kx) and channel c.  w_perm may be NULL for one group
 *              (row j writes output column j).  MXFP4 x MXFP4 groups are
 *              MXQ_ERR_UNSUPPORTED (the scaled-MFMA route has no im2col
 *              reader).
 *  bias, out, ld_out, n_out, workspace  as in mxq_gemm_mixed; out row m is
 *              output pixel m (same order as x).  No low-rank branch.
 * Output pixel (y, x) with tap (ky, kx) reads input pixel (y + ky - 1,
 * x + kx - 1) of the same image, and zero where that lies outside it.
 */
mxq_status mxq_conv3x3_gemm_mixed(const mxq_qtensor* x, int64_t height, int64_t width,
                                  const mxq_qtensor* w_groups, int32_t n_groups,
                                  const int32_t* w_perm, const void* bias, void* out,
                                  int64_t ld_out, int64_t n_out, void* workspace,
                                  size_t ws_bytes, void* stream);

/*
 * mxq_quantize_mse -- quantize weights [rows, cols] to MXFP4 or NVFP4 with
 * least-squared-error scales instead of the amax rule ("Bridging the Gap
 * ... Microscaling FP4 Quantization" summary, MR-GPTQ modification 1: the
 * grid is chosen for least MSE by optimising block and tensor scales in
 * turn).  Weight preparation, once per layer.
 *
 * Block step: each block's scale code is, among every code of its format
 * (E8M0 0..254; E4M3 0..126 times g), the one whose squared error
 * sum_i (x_i - x_hat_i)^2 -- taken over the block in element order, each
 * subtraction, product and addition rounded to float64 separately -- is
 * smallest, ties to the smaller code; elements then round to nearest even
 * under that scale.  NVFP4 adds a tensor step: with the codes fixed,
 * g = RN_fp32(P / Q), P = sum x w, Q = sum w^2 (w = element value times its
 * block scale), float64 sums of row sums taken in order (Q = 0, or a
 * quotient that rounds to zero, keeps g).  Rounds: NVFP4 amax-rule g, block
 * step, tensor step, block step (g written to *out->tensor_scale); MXFP4
 * one block step.  Never a larger total squared error than the amax rule.
 *
 *  w, dtype, ldw   as mxq_quantize's x (fp32 or bf16, 16-byte aligned).
 *  out         out->fmt MXQ_FMT_MXFP4 or MXQ_FMT_NVFP4 (others:
 *              MXQ_ERR_UNSUPPORTED); buffers as for mxq_quantize.
 *  workspace   mxq_workspace_size(MXQ_OP_QUANTIZE_MSE, rows, cols, fmt)
 *              bytes, 16-byte aligned (none for MXFP4).
 * cols must be a multiple of 32.
 */
mxq_status mxq_quantize_mse(const void* w, int32_t dtype, int64_t rows, int64_t cols,
                            int64_t ldw, mxq_qtensor* out, void* workspace, size_t ws_bytes,
                            void* stream);

/*
 * mxq_lowrank_split -- offline SVDQuant split of a weight (Nunchaku article,
 * "main explanation": the hardest part of the weight is kept as a low-rank
 * 16-bit branch and the rest is quantized to 4 bits):
 *   W [n][k] ~= (L1 L2)^T + R,  L1 = V_r sqrt(S_r) [k][r],  L2 = sqrt(S_r) U_r^T [r][n],
 * from the rank-r truncated SVD W_r = U_r S_r V_r^T, factors rounded to
 * bf16, R = W - (L1 L2)^T in fp32 (then quantize R with mxq_quantize or
 * mxq_quantize_mse).  The subspace comes from `iters` rounds of subspace
 * iteration from a fixed start (r + 16 columns) and a Rayleigh-Ritz step
 * (float64 Jacobi); it converges to the truncated SVD when sigma_r is well
 * above sigma_{r+17}.  Singular pairs carry an arbitrary sign; L1 L2 and R do
 * not depend on it.  Weight preparation, once per layer.
 *
 *  w           device fp32 [n][ldw] (k columns used), 4-byte aligned.
 *  rank        1..128, at most min(n, k).   iters  0 (default 8) .. 64.
 *  l1t         device bf16 [rank][k]: L1^T, the layout mxq_quantize's
 *              lr_l1t takes.
 *  l2t         device bf16 [n][rank]: L2^T, the layout mxq_gemm's lr_l2t takes.
 *  resid       device fp32 [n][ld_resid]: R.
 *  sigma       optional device fp32 [rank]: the singular values, decreasing.
 *  workspace   mxq_workspace_size(MXQ_OP_LOWRANK_SPLIT, n, k, rank) bytes,
 *              256-byte aligned.
 */
mxq_status mxq_lowrank_split(const float* w, int64_t n, int64_t k, int64_t ldw, int32_t rank,
                             int32_t iters, void* l1t, void* l2t, float* resid, int64_t ld_resid,
                             float* sigma, void* workspace, size_t ws_bytes, void* stream);

/*
 * mxq_select_format -- per-output-channel weight format by least
 * reconstruction error (Chameleon article, "the format is chosen by the
 * value distribution").
 *
 *  w           device fp32 or bf16 weights [n][ldw], k columns used.
 *  candidates  host array of n_cand formats (MXQ_FMT_INT4 / MXFP4 / NVFP4),
 *              in tie-break order (earliest wins a tie).
 *  choice_out  device uint8[n]: index into candidates of the chosen format.
 *  sse_out     optional device float64 [n][n_cand]: sum over the row of
 *              (w - dequant(quant(w)))^2, each squared difference exact.
 *  perm_out    optional device int32[n]: rows grouped by chosen candidate in
 *              candidate order, ascending row index inside a group.
 *  counts_out  optional device int32[n_cand]: rows per candidate.
 *  g_out       optional device float: the NVFP4 tensor scale over all of w
 *              (the one the NVFP4 candidate used).
 *  workspace   mxq_workspace_size(MXQ_OP_SELECT, n, k, 0) bytes.
 * k must be a multiple of 32.
 */
mxq_status mxq_select_format(const void* w, int32_t dtype, int64_t n, int64_t k, int64_t ldw,
                             const int32_t* candidates, int32_t n_cand,
                             uint8_t* choice_out, double* sse_out, int32_t* perm_out,
                             int32_t* counts_out, float* g_out,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * mxq_act_format_for_step -- host-only table read (Chameleon article: ten
 * trajectory intervals; at inference routing is a table read).
 * bucket = min(n_buckets - 1, floor(n_buckets * step / num_steps));
 * returns table[layer * n_buckets + bucket], or -1 for invalid arguments
 * (NULL table, layer outside [0, n_layers), step outside [0, num_steps)).
 */
int32_t mxq_act_format_for_step(const uint8_t* table, int32_t n_layers, int32_t n_buckets,
                                int32_t layer, int32_t step, int32_t num_steps);

/* Operations for mxq_workspace_size. */
enum { MXQ_OP_QUANTIZE = 1, MXQ_OP_GEMM = 2, MXQ_OP_SELECT = 3, MXQ_OP_QUANTIZE_MSE = 4,
       MXQ_OP_LOWRANK_SPLIT = 5 };

/* Workspace bytes an operation needs for a [rows, cols] operand of format
 * fmt (0 when none); for MXQ_OP_GEMM rows = M, cols = N (weight rows) and
 * fmt = the weight format (the optional split-K workspace); for
 * MXQ_OP_LOWRANK_SPLIT rows = n, cols = k and fmt = the rank.  Returns -1 for
 * unknown arguments.  Host-only. */
int64_t mxq_workspace_size(int32_t op, int64_t rows, int64_t cols, int32_t fmt);

/* Per-row storage of a format with cols elements per row: code bytes and
 * scale bytes (the minimum ld_codes / ld_scales).  Returns MXQ_ERR_SHAPE if
 * cols is not a multiple of the format's block.  Host-only. */
mxq_status mxq_storage(int32_t fmt, int64_t cols, int64_t* code_bytes, int64_t* scale_bytes);

/* Static description of a status code.  Host-only. */
const char* mxq_status_string(int32_t status);

/* MXQ_VERSION of the built library.  Host-only. */
int32_t mxq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
