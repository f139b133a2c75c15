// Offline SVDQuant split of a weight (Nunchaku / SVDQuant article, "main
// explanation": the hardest part of the weight is kept as a low-rank 16-bit
// branch, the rest is quantized to 4 bits): W [N][K] ~= (L1 L2)^T + R with
// the rank-r truncated SVD W_r = U_r S_r V_r^T, L1 = V_r sqrt(S_r),
// L2 = sqrt(S_r) U_r^T (bf16) and R = W - (L1 L2)^T (fp32).
//
// The top-r singular subspace comes from subspace iteration on the GPU:
// starting from a fixed +-1 block Z [K][p] (p = r + 16 columns, made even),
// each round forms Y = W Z, orthonormalises it (Cholesky QR, twice), forms
// Z = W^T Q and orthonormalises that; a Rayleigh-Ritz step then takes the
// eigen-decomposition of (Q^T W)(Q^T W)^T (cyclic Jacobi in float64) for the
// singular values and both singular bases.  All products are fp32 FMAs
// (exact operands, fp32 accumulation); Gram matrices, Cholesky and Jacobi
// run in float64.  This is weight preparation, run once per layer.
#include <hip/hip_bf16.h>

#include "device_common.h"
#include "kernels.h"

namespace mxq {
namespace {

// C [M][P] (row stride ldc) = sum_k A(m, k) B(k, p), with A(m, k) =
// a[m * sam + k * sak] and B(k, p) = b[k * sbk + p * sbp]; 64 x 64 tiles,
// 16-deep K chunks through LDS, 4 x 4 outputs per thread.
__global__ __launch_bounds__(256) void sgemm_kernel(const float* a, int64_t sam, int64_t sak,
                                                    const float* b, int64_t sbk, int64_t sbp,
                                                    float* c, int64_t ldc, int64_t M,
                                                    int64_t K, int64_t P) {
  __shared__ float as[16][64 + 1];
  __shared__ float bs[16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 64, p0 = (int64_t)blockIdx.x * 64;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += 16) {
    for (int t = threadIdx.x; t < 16 * 64; t += 256) {
      const int kk = t / 64, mm = t % 64;
      const int64_t m = m0 + mm, k = k0 + kk;
      as[kk][mm] = (m < M && k < K) ? a[m * sam + k * sak] : 0.f;
      const int64_t p = p0 + mm;
      bs[kk][mm] = (p < P && k < K) ? b[k * sbk + p * sbp] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = as[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = m0 + ty * 4 + i, p = p0 + tx * 4 + j;
      if (m < M && p < P) c[m * ldc + p] = acc[i][j];
    }
}

// G [p][p] (float64) = sum_n X(n, i) X(n, j), X(n, i) = x[n * sxn + i * sxi];
// one thread per entry of a 16 x 16 tile of G, reducing over all n in order.
__global__ __launch_bounds__(256) void gram_kernel(const float* x, int64_t sxn, int64_t sxi,
                                                   int64_t rows, int p, double* g) {
  const int i = blockIdx.y * 16 + (threadIdx.x >> 4), j = blockIdx.x * 16 + (threadIdx.x & 15);
  if (i >= p || j >= p) return;
  double s = 0.0;
  for (int64_t n = 0; n < rows; ++n)
    s += (double)x[n * sxn + i * sxi] * (double)x[n * sxn + j * sxi];
  g[(int64_t)i * p + j] = s;
}

// Cholesky G = L L^T (one workgroup, float64), then T = L^-T as fp32, so
// that Q = Y T has orthonormal columns.  A pivot that is not positive (a
// rank-deficient block) gives a zero column of T: that direction is dropped.
__global__ __launch_bounds__(256) void chol_inv_kernel(double* g, int p, double* linv, float* t) {
  // g is overwritten by L (lower triangle)
  for (int j = 0; j < p; ++j) {
    __shared__ double d;
    if (threadIdx.x == 0) {
      double s = g[(int64_t)j * p + j];
      for (int k = 0; k < j; ++k) s -= g[(int64_t)j * p + k] * g[(int64_t)j * p + k];
      d = s > 0.0 ? sqrt(s) : 0.0;
      g[(int64_t)j * p + j] = d;
    }
    __syncthreads();
    for (int i = j + 1 + threadIdx.x; i < p; i += blockDim.x) {
      double s = g[(int64_t)i * p + j];
      for (int k = 0; k < j; ++k) s -= g[(int64_t)i * p + k] * g[(int64_t)j * p + k];
      g[(int64_t)i * p + j] = d > 0.0 ? s / d : 0.0;
    }
    __syncthreads();
  }
  // columns of L^-1 by forward substitution (one thread per column)
  for (int c = threadIdx.x; c < p; c += blockDim.x) {
    for (int i = 0; i < p; ++i) {
      double s = (i == c) ? 1.0 : 0.0;
      for (int k = c; k < i; ++k) s -= g[(int64_t)i * p + k] * linv[(int64_t)k * p + c];
      const double di = g[(int64_t)i * p + i];
      linv[(int64_t)i * p + c] = (i < c || di <= 0.0) ? 0.0 : s / di;
    }
  }
  __syncthreads();
  // T = (L^-1)^T: T[k][i] = Linv[i][k]
  for (int e = threadIdx.x; e < p * p; e += blockDim.x) {
    const int k = e / p, i = e % p;
    t[e] = (float)linv[(int64_t)i * p + k];
  }
}

// Cyclic Jacobi on the symmetric a [p][p] (float64, overwritten): round-robin
// pairs, p2/2 disjoint rotations per step (p2 = p rounded up to even; the
// extra index sits out).  Eigenvectors accumulate in v [p][p]; then the
// eigenpairs are sorted by decreasing eigenvalue into e (fp32 [p][p],
// columns) and sigma = sqrt(max(lambda, 0)).
__global__ __launch_bounds__(1024) void jacobi_kernel(double* a, double* v, int p, float* e,
                                                      float* sigma, int sweeps) {
  __shared__ int pi[256], pj[256];
  __shared__ double cs[128], sn[128];
  __shared__ int order[256];
  const int p2 = (p + 1) & ~1, half = p2 / 2;
  for (int idx = threadIdx.x; idx < p * p; idx += blockDim.x)
    v[idx] = (idx / p == idx % p) ? 1.0 : 0.0;
  // round-robin tournament: position 0 fixed, the others rotate
  __shared__ int pos[256];
  for (int idx = threadIdx.x; idx < p2; idx += blockDim.x) pos[idx] = idx;
  __syncthreads();
  for (int sw = 0; sw < sweeps; ++sw) {
    for (int step = 0; step < p2 - 1; ++step) {
      for (int k = threadIdx.x; k < half; k += blockDim.x) {
        int i = pos[k], j = pos[p2 - 1 - k];
        if (i > j) { const int t = i; i = j; j = t; }
        pi[k] = i;
        pj[k] = j;
        double c = 1.0, s = 0.0;
        if (j < p) {
          const double aij = a[(int64_t)i * p + j];
          if (aij != 0.0) {
            const double aii = a[(int64_t)i * p + i], ajj = a[(int64_t)j * p + j];
            const double theta = (ajj - aii) / (2.0 * aij);
            const double tt = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
            c = 1.0 / sqrt(tt * tt + 1.0);
            s = tt * c;
          }
        }
        cs[k] = c;
        sn[k] = s;
      }
      __syncthreads();
      // rows i, j of a (every column)
      for (int idx = threadIdx.x; idx < half * p; idx += blockDim.x) {
        const int k = idx / p, m = idx % p, i = pi[k], j = pj[k];
        if (j >= p) continue;
        const double c = cs[k], s = sn[k];
        const double ai = a[(int64_t)i * p + m], aj = a[(int64_t)j * p + m];
        a[(int64_t)i * p + m] = c * ai - s * aj;
        a[(int64_t)j * p + m] = s * ai + c * aj;
      }
      __syncthreads();
      // columns i, j of a and v (every row)
      for (int idx = threadIdx.x; idx < half * p; idx += blockDim.x) {
        const int k = idx / p, m = idx % p, i = pi[k], j = pj[k];
        if (j >= p) continue;
        const double c = cs[k], s = sn[k];
        const double ai = a[(int64_t)m * p + i], aj = a[(int64_t)m * p + j];
        a[(int64_t)m * p + i] = c * ai - s * aj;
        a[(int64_t)m * p + j] = s * ai + c * aj;
        const double vi = v[(int64_t)m * p + i], vj = v[(int64_t)m * p + j];
        v[(int64_t)m * p + i] = c * vi - s * vj;
        v[(int64_t)m * p + j] = s * vi + c * vj;
      }
      __syncthreads();
      // next pairing: keep pos[0], rotate the rest by one
      if (threadIdx.x == 0) {
        const int last = pos[p2 - 1];
        for (int q = p2 - 1; q > 1; --q) pos[q] = pos[q - 1];
        pos[1] = last;
      }
      __syncthreads();
    }
  }
  // order by decreasing eigenvalue (rank by counting; ties by index)
  for (int i = threadIdx.x; i < p; i += blockDim.x) {
    const double li = a[(int64_t)i * p + i];
    int rank = 0;
    for (int j = 0; j < p; ++j) {
      const double lj = a[(int64_t)j * p + j];
      rank += (lj > li) || (lj == li && j < i);
    }
    order[rank] = i;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < p * p; idx += blockDim.x) {
    const int m = idx / p, col = idx % p;
    e[idx] = (float)v[(int64_t)m * p + order[col]];
  }
  for (int col = threadIdx.x; col < p; col += blockDim.x) {
    const double l = a[(int64_t)order[col] * p + order[col]];
    sigma[col] = (float)sqrt(l > 0.0 ? l : 0.0);
  }
}

// The fixed +-1 start block: the sign of a 32-bit integer hash of (k, j).
__global__ __launch_bounds__(256) void start_kernel(float* z, int64_t rows, int p) {
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < rows * p;
       idx += (int64_t)gridDim.x * 256) {
    uint32_t h = (uint32_t)idx * 0x9E3779B1u;
    h ^= h >> 15;
    h *= 0x85EBCA77u;
    h ^= h >> 13;
    z[idx] = (h & 0x10000u) ? 1.f : -1.f;
  }
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// L1^T [r][K] = bf16(sqrt(sigma_j) V[k][j]) with V = (B^T E) / sigma (here
// bte = B^T E, [K][p]); L2^T [N][r] = bf16(sqrt(sigma_j) U[n][j]), U = Q E.
// A singular value that is zero gives zero factors.
__global__ __launch_bounds__(256) void factors_kernel(const float* bte, const float* u,
                                                      const float* sigma, int64_t n, int64_t k,
                                                      int p, int r, uint16_t* l1t, uint16_t* l2t) {
  const int64_t tot1 = (int64_t)r * k, tot = tot1 + n * r;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < tot;
       idx += (int64_t)gridDim.x * 256) {
    if (idx < tot1) {
      const int j = (int)(idx / k);
      const int64_t kk = idx % k;
      const float s = sigma[j];
      l1t[idx] = to_bf16(s > 0.f ? bte[kk * p + j] / sqrtf(s) : 0.f);
    } else {
      const int64_t e = idx - tot1, nn = e / r;
      const int j = (int)(e % r);
      const float s = sigma[j];
      l2t[e] = to_bf16(s > 0.f ? sqrtf(s) * u[nn * p + j] : 0.f);
    }
  }
}

// R [N][K] = W - L2^T L1^T (bf16 products exact in fp32, summed over the
// rank in order).
__global__ __launch_bounds__(256) void residual_kernel(const float* w, int64_t ldw,
                                                       const uint16_t* l1t, const uint16_t* l2t,
                                                       int64_t n, int64_t k, int r, float* res,
                                                       int64_t ldr) {
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n * k;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t row = idx / k, col = idx % k;
    float s = 0.f;
    for (int j = 0; j < r; ++j)
      s = __builtin_fmaf(bf16_bits_to_f32(l2t[row * r + j]), bf16_bits_to_f32(l1t[(int64_t)j * k + col]), s);
    res[row * ldr + col] = w[row * ldw + col] - s;
  }
}

struct Ws {
  float *z, *y, *q, *t, *b, *e, *sigma, *bte;
  double *g, *linv, *v;
};

int split_cols(int r, int64_t n, int64_t k) {
  int64_t p = r + 16;
  p = (p + 1) & ~1;
  const int64_t mn = n < k ? n : k;
  return (int)(p < mn ? p : mn);
}

Ws carve(void* base, int64_t n, int64_t k, int p) {
  char* c = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* r = c;
    c += (bytes + 255) & ~(size_t)255;
    return r;
  };
  Ws w;
  w.g = reinterpret_cast<double*>(take((size_t)p * p * 8));
  w.linv = reinterpret_cast<double*>(take((size_t)p * p * 8));
  w.v = reinterpret_cast<double*>(take((size_t)p * p * 8));
  w.z = reinterpret_cast<float*>(take((size_t)k * p * 4));
  w.y = reinterpret_cast<float*>(take((size_t)n * p * 4));
  w.q = reinterpret_cast<float*>(take((size_t)n * p * 4));
  w.t = reinterpret_cast<float*>(take((size_t)p * p * 4));
  w.b = reinterpret_cast<float*>(take((size_t)p * k * 4));
  w.e = reinterpret_cast<float*>(take((size_t)p * p * 4));
  w.sigma = reinterpret_cast<float*>(take((size_t)p * 4));
  w.bte = reinterpret_cast<float*>(take((size_t)k * p * 4));
  return w;
}

hipError_t sgemm(const float* a, int64_t sam, int64_t sak, const float* b, int64_t sbk,
                 int64_t sbp, float* c, int64_t ldc, int64_t M, int64_t K, int64_t P,
                 hipStream_t s) {
  const dim3 grid((unsigned)((P + 63) / 64), (unsigned)((M + 63) / 64));
  sgemm_kernel<<<grid, 256, 0, s>>>(a, sam, sak, b, sbk, sbp, c, ldc, M, K, P);
  return hipGetLastError();
}

// Orthonormal columns of x [rows][p] into out (Cholesky QR).
hipError_t orth(const float* x, int64_t rows, int p, float* out, const Ws& w, hipStream_t s) {
  const dim3 gg((unsigned)((p + 15) / 16), (unsigned)((p + 15) / 16));
  gram_kernel<<<gg, 256, 0, s>>>(x, p, 1, rows, p, w.g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  chol_inv_kernel<<<1, 256, 0, s>>>(w.g, p, w.linv, w.t);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return sgemm(x, p, 1, w.t, p, 1, out, p, rows, p, p, s);
}

// Cholesky QR twice (the second pass restores orthogonality lost to rounding).
hipError_t orth2(float* x, int64_t rows, int p, float* tmp, const Ws& w, hipStream_t s) {
  hipError_t e = orth(x, rows, p, tmp, w, s);
  if (e != hipSuccess) return e;
  return orth(tmp, rows, p, x, w, s);
}

}  // namespace

int64_t lowrank_split_workspace(int64_t n, int64_t k, int r) {
  const int p = split_cols(r, n, k);
  auto up = [](int64_t b) { return (b + 255) & ~(int64_t)255; };
  return 3 * up((int64_t)p * p * 8) + up(k * p * 4) + 2 * up(n * p * 4) + up((int64_t)p * p * 4) +
         up((int64_t)p * k * 4) + up((int64_t)p * p * 4) + up((int64_t)p * 4) + up(k * p * 4);
}

hipError_t launch_lowrank_split(const LowrankSplitArgs& a, hipStream_t s) {
  const int64_t n = a.n, k = a.k;
  const int r = a.rank, p = split_cols(r, n, k);
  const Ws w = carve(a.ws, n, k, p);
  hipError_t e;
  start_kernel<<<256, 256, 0, s>>>(w.z, k, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = orth2(w.z, k, p, w.bte, w, s)) != hipSuccess) return e;
  for (int it = 0; it < a.iters; ++it) {
    // Y = W Z, Q = orth(Y); Z = W^T Q, Z = orth(Z)
    if ((e = sgemm(a.w, a.ldw, 1, w.z, p, 1, w.y, p, n, k, p, s)) != hipSuccess) return e;
    if ((e = orth2(w.y, n, p, w.q, w, s)) != hipSuccess) return e;
    if ((e = sgemm(a.w, 1, a.ldw, w.y, p, 1, w.z, p, k, n, p, s)) != hipSuccess) return e;
    if ((e = orth2(w.z, k, p, w.bte, w, s)) != hipSuccess) return e;
  }
  // Rayleigh-Ritz: Q = orth(W Z), B = Q^T W [p][K], B B^T = E diag(lambda) E^T
  if ((e = sgemm(a.w, a.ldw, 1, w.z, p, 1, w.y, p, n, k, p, s)) != hipSuccess) return e;
  if ((e = orth2(w.y, n, p, w.q, w, s)) != hipSuccess) return e;   // Q is in w.y
  if ((e = sgemm(w.y, 1, p, a.w, a.ldw, 1, w.b, k, p, n, k, s)) != hipSuccess) return e;
  const dim3 gg((unsigned)((p + 15) / 16), (unsigned)((p + 15) / 16));
  gram_kernel<<<gg, 256, 0, s>>>(w.b, 1, k, k, p, w.g);   // (B B^T)[i][j] = sum_k B[i][k] B[j][k]
  if ((e = hipGetLastError()) != hipSuccess) return e;
  jacobi_kernel<<<1, 1024, 0, s>>>(w.g, w.v, p, w.e, w.sigma, 12);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // U = Q E [N][p] (into w.q), B^T E [K][p]
  if ((e = sgemm(w.y, p, 1, w.e, p, 1, w.q, p, n, p, p, s)) != hipSuccess) return e;
  if ((e = sgemm(w.b, 1, k, w.e, p, 1, w.bte, p, k, p, p, s)) != hipSuccess) return e;
  factors_kernel<<<1024, 256, 0, s>>>(w.bte, w.q, w.sigma, n, k, p, r, a.l1t, a.l2t);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.sigma) {
    if ((e = hipMemcpyAsync(a.sigma, w.sigma, (size_t)r * 4, hipMemcpyDeviceToDevice, s)) !=
        hipSuccess)
      return e;
  }
  residual_kernel<<<4096, 256, 0, s>>>(a.w, a.ldw, a.l1t, a.l2t, n, k, r, a.resid, a.ld_resid);
  return hipGetLastError();
}

}  // namespace mxq
