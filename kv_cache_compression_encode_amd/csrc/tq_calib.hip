// Calibration moments of the SpectralQuant rotation on the device ([SQ]
// tweet 4: the per-head eigenbasis of the key covariance, from a short
// calibration pass over a couple of thousand tokens).
//
// Per head h of n calibration vectors x_t of d coordinates (fp32 or bf16):
//   sum_x[h][i]    = sum_t x_ti
//   mom_x[h][i][k] = sum_t x_ti x_tk
//   mom_u[h][i][k] = sum_t x_ti x_tk / ||x_t||^2      (0 for a zero vector)
// all in fp64: the inputs and their pairwise products are exact in fp64, so
// only the sums round.  The host then forms the centred covariance
// mom_x / n - mean mean^T, its eigenbasis Pi (a 128 x 128 eigensolve per
// head), and sigma_i^2 = p_i^T mom_u p_i / n with p_i row i of Pi, the mean
// square of rotated coordinate i of the normalised vectors.
//
// The contraction runs on the fp64 vector unit: on MI355X the fp64 matrix
// cores have the same peak rate as fp64 vector FMAs, and at this size (a few
// hundred MFLOP) the launch and the copies dominate either way.
#include <hip/hip_runtime.h>

#include "tq_kernels.h"

namespace tq {
namespace {

__device__ __forceinline__ double calib_elem(const void* x, int bf16, int64_t e) {
  if (bf16) return double(__uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[e]) << 16));
  return double(static_cast<const float*>(x)[e]);
}

// One wave per vector: 1 / ||x_t||^2, or 0 for a zero vector.
__global__ __launch_bounds__(256) void calib_rnorm_kernel(const void* x, int bf16, int64_t rows, int d,
                                                          double* rinv2) {
  const int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  double s = 0.0;
  for (int i = lane; i < d; i += 64) {
    const double v = calib_elem(x, bf16, r * d + i);
    s = fma(v, v, s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) rinv2[r] = s > 0.0 ? 1.0 / s : 0.0;
}

// Block (tile, head): the 32 x 32 output tile (ti, tk) of both moment
// matrices; thread (a, c) owns rows 2a, 2a + 1 and columns 2c, 2c + 1 of it.
// The vectors stream through LDS 32 at a time (the tile's two 32-column
// slices of each).  Tiles with tk = 0 also form the column sums of their rows.
constexpr int kCT = 32;  // output tile edge and vectors per LDS stage
__global__ __launch_bounds__(256) void calib_moments_kernel(const void* x, int bf16, int64_t n, int d,
                                                            const double* rinv2, double* mom_x,
                                                            double* mom_u, double* sum_x) {
  const int nt = d / kCT;
  const int ti = blockIdx.x / nt, tk = blockIdx.x % nt;
  const int h = blockIdx.y;
  const int t = threadIdx.x, a = t >> 4, c = t & 15;
  __shared__ double sa[kCT][kCT + 1], sb[kCT][kCT + 1], sw[kCT];
  const int64_t base = int64_t(h) * n;
  double ax[2][2] = {{0.0, 0.0}, {0.0, 0.0}}, au[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
  double sx0 = 0.0, sx1 = 0.0;
  for (int64_t r0 = 0; r0 < n; r0 += kCT) {
    for (int e = t; e < kCT * kCT; e += blockDim.x) {
      const int rr = e / kCT, cc = e % kCT;
      const int64_t row = r0 + rr;
      const bool ok = row < n;
      sa[rr][cc] = ok ? calib_elem(x, bf16, (base + row) * d + ti * kCT + cc) : 0.0;
      sb[rr][cc] = ok ? calib_elem(x, bf16, (base + row) * d + tk * kCT + cc) : 0.0;
    }
    if (t < kCT) sw[t] = r0 + t < n ? rinv2[base + r0 + t] : 0.0;
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < kCT; ++rr) {
      const double a0 = sa[rr][2 * a], a1 = sa[rr][2 * a + 1];
      const double b0 = sb[rr][2 * c], b1 = sb[rr][2 * c + 1];
      const double w = sw[rr];
      const double p00 = a0 * b0, p01 = a0 * b1, p10 = a1 * b0, p11 = a1 * b1;
      ax[0][0] += p00;
      ax[0][1] += p01;
      ax[1][0] += p10;
      ax[1][1] += p11;
      au[0][0] = fma(p00, w, au[0][0]);
      au[0][1] = fma(p01, w, au[0][1]);
      au[1][0] = fma(p10, w, au[1][0]);
      au[1][1] = fma(p11, w, au[1][1]);
      sx0 += a0;
      sx1 += a1;
    }
    __syncthreads();
  }
  const int i0 = ti * kCT + 2 * a, k0 = tk * kCT + 2 * c;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const size_t e = (size_t(h) * d + i0 + u) * d + k0 + v;
      mom_x[e] = ax[u][v];
      mom_u[e] = au[u][v];
    }
  if (tk == 0 && c == 0) {
    sum_x[size_t(h) * d + i0] = sx0;
    sum_x[size_t(h) * d + i0 + 1] = sx1;
  }
}

}  // namespace

hipError_t launch_calib_moments(const void* x, int bf16, int heads, int64_t n, int d, double* rinv2,
                                double* mom_x, double* mom_u, double* sum_x, hipStream_t s) {
  if (d % kCT != 0 || heads < 1 || n < 1) return hipErrorInvalidValue;
  const int64_t rows = int64_t(heads) * n;
  hipLaunchKernelGGL(calib_rnorm_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s, x, bf16, rows, d,
                     rinv2);
  const int nt = d / kCT;
  hipLaunchKernelGGL(calib_moments_kernel, dim3(unsigned(nt * nt), unsigned(heads)), dim3(256), 0, s, x, bf16, n,
                     d, rinv2, mom_x, mom_u, sum_x);
  return hipGetLastError();
}

}  // namespace tq
