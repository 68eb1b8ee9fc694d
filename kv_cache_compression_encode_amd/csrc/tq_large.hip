// TurboQuant encode and scoring for wide vectors (d a multiple of 128, e.g.
// the 1536-dim vector-search workload).  At this width the rotation
// Y = X Pi^T, the QJL sketch Z = R S^T and the scoring Q' K_hat^T are plain
// dense GEMMs over whole rows, so they run as rocBLAS fp16 GEMMs with fp32
// accumulation.  fp32 accuracy comes from hi/lo fp16 splits laid side by side
// along the reduction axis: [a_hi | a_hi | a_lo] . [b_hi | b_lo | b_hi]^T =
// a_hi b_hi + a_hi b_lo + a_lo b_hi, one GEMM per product (the sketch S is
// stored in fp16, so there [r_hi | r_lo] . [S | S]^T suffices).  The per-element
// steps in between are the kernels below:
//   rowprep   : n_x, per-row power-of-two scale, split of x;
//   quantize  : Lloyd-Max index per coordinate (TurboQuant paper review,
//               "Method"), row-layout bit planes, residual r = y - c[idx]
//               split for the sketch GEMM, ||r||^2;
//   signpack  : sign bits [z >= 0] and the fp16 norms;
//   dequant   : key rows [c[idx] | +-n_r] (fp16) of stored records;
//   qsplit    : query rows [q' | sqrt(pi/2)/m q_s] scaled by a power of two
//               into fp16 (a 2^-12 relative rounding: score error at most
//               2^-12 ||q'|| ||k_hat||, far inside the 1e-3 tolerance);
//   combine   : s = n_x part / query scale.
// Rows are processed in chunks so the workspace stays bounded.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <cmath>
#include <mutex>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr float kQjl = 1.2533141373155001f;  // sqrt(pi / 2)

__device__ __forceinline__ uint16_t f16b(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ float f16v(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }

// One wave per row: n_x, scale 2^e putting max|x| in [2^14, 2^15), and the
// row [hi | hi | lo] of x 2^e in fp16 (xcat, [rows][3d]).  w[row] = 16 2^e n_x
// relates the GEMM output (with 16 Pi) to the rotated unit vector.
__global__ __launch_bounds__(256) void rowprep_kernel(const void* x, int x_bf16, int64_t ld,
                                                      int64_t rows, int d, uint16_t* xcat, float* w,
                                                      float* nx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  auto at = [&](int i) -> float {
    if (x_bf16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[row * ld + i]) << 16);
    return static_cast<const float*>(x)[row * ld + i];
  };
  float mx = 0.f;
  for (int i = lane; i < d; i += 64) mx = fmaxf(mx, fabsf(at(i)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const int ebits = int((__float_as_uint(mx) >> 23) & 0xff);
  const float p2 = mx > 0.f ? __uint_as_float(uint32_t(min(253, max(1, 268 - ebits))) << 23) : 1.f;
  // the squares are summed over x 2^e, so none underflows whatever the
  // row's magnitude (the scaling is exact: n_x is the same for ordinary rows)
  float ss = 0.f;
  uint16_t* out = xcat + row * 3 * d;
  for (int i = lane; i < d; i += 64) {
    const float v = at(i) * p2;
    ss = fmaf(v, v, ss);
    const uint16_t h = f16b(v);
    out[i] = h;
    out[d + i] = h;
    out[2 * d + i] = f16b(v - f16v(h));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) {
    const float n = sqrtf(ss) / p2;
    nx[row] = n;
    w[row] = 16.f * p2 * (n > 0.f ? n : 1.f);
  }
}

// [rows][3 cols] = [hi | lo | hi] of a pair of fp16 matrices [rows][cols]
// (lo == nullptr: [rows][2 cols] = [hi | hi]).
__global__ void cat3_kernel(const uint16_t* hi, const uint16_t* lo, int64_t rows, int cols,
                            uint16_t* out) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= rows * cols) return;
  const int64_t r = e / cols;
  const int c = int(e % cols);
  if (!lo) {
    uint16_t* o = out + r * 2 * cols;
    o[c] = hi[e];
    o[cols + c] = hi[e];
    return;
  }
  uint16_t* o = out + r * 3 * cols;
  o[c] = hi[e];
  o[cols + c] = lo[e];
  o[2 * cols + c] = hi[e];
}

// One wave per row, 64 coordinates per step (lane = coordinate): index by the
// thresholds (scaled by w[row] instead of dividing y), bit planes by ballot,
// residual r = y - c[idx] split into rcat [rows][2m] = [hi | lo] of 32 r,
// and ||r||^2 by a wave reduction.  Rows >= rows_valid (padding of the last
// tile) get zero records.
__global__ __launch_bounds__(256) void quantize_kernel(CodecView cv, const float* y, const float* w,
                                                       const float* nx, int64_t row0, int64_t rows,
                                                       int64_t rows_valid, uint8_t* rec, uint16_t* rcat,
                                                       float* rr) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int d = cv.d, ub = cv.ubits, nthr = (1 << ub) - 1;
  const bool prod = cv.mode == TQ_PROD;
  const int64_t grow = row0 + row;
  uint8_t* trec = rec + (grow / kTile) * cv.tile_bytes;
  const int slot = int(grow % kTile);
  const bool valid = row < rows_valid;
  const float wr = valid ? w[row] : 1.f;
  const float inv = 1.f / wr;
  float thr[kMaxLevels - 1];
#pragma unroll
  for (int t = 0; t < kMaxLevels - 1; ++t) thr[t] = cv.uthr[t] * wr;
  float rsum = 0.f;
  for (int j = 0; j < d / 64; ++j) {
    const int dim = 64 * j + lane;
    int idx = 0;
    float c = cv.ucen[0];
    float v = 0.f;
    if (valid) {
      v = y[row * d + dim];
#pragma unroll
      for (int t = 0; t < kMaxLevels - 1; ++t)
        if (t < nthr && v >= thr[t]) { idx = t + 1; c = cv.ucen[t + 1]; }
    }
    if (prod && valid && dim < cv.m) {
      const float r = v * inv - c;
      rsum = fmaf(r, r, rsum);
      const float rs = 32.f * r;
      const uint16_t h = f16b(rs);
      uint16_t* o = rcat + row * 2 * cv.m;
      o[dim] = h;
      o[cv.m + dim] = f16b(rs - f16v(h));
    }
    for (int p = 0; p < ub; ++p) {
      const uint64_t mask = __ballot((idx >> p) & 1);
      if (lane < 2) {
        const int byte = p * (d / 8) + 8 * j + 4 * lane;  // position in the row bit string
        *reinterpret_cast<uint32_t*>(trec + size_t(byte / 16) * kTile * 16 + size_t(slot) * 16 + byte % 16) =
            uint32_t(mask >> (32 * lane));
      }
    }
  }
  if (prod) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rsum += __shfl_xor(rsum, o, 64);
    if (lane == 0) rr[row] = rsum;
  }
  if (lane == 0) *reinterpret_cast<uint16_t*>(trec + cv.off_nx + 2 * slot) = valid ? f16b(nx[row]) : uint16_t(0);
}

// One wave per row: sign bits [z >= 0] by ballot (64 per step) and n_r.
__global__ __launch_bounds__(256) void signpack_kernel(CodecView cv, const float* z, const float* rr,
                                                       int64_t row0, int64_t rows, int64_t rows_valid,
                                                       uint8_t* rec) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int m = cv.m;
  const int64_t grow = row0 + row;
  uint8_t* trec = rec + (grow / kTile) * cv.tile_bytes;
  const int slot = int(grow % kTile);
  const bool valid = row < rows_valid;
  for (int j = 0; j < m / 64; ++j) {
    const bool bit = valid && z[row * m + 64 * j + lane] >= 0.f;
    const uint64_t mask = __ballot(bit);
    if (lane < 2) {
      const int byte = 8 * j + 4 * lane;  // all sign chunks are 16 bytes wide (m % 128 == 0)
      *reinterpret_cast<uint32_t*>(trec + cv.off_signs + size_t(byte / 16) * kTile * 16 + size_t(slot) * 16 +
                                   byte % 16) = uint32_t(mask >> (32 * lane));
    }
  }
  if (lane == 0)
    *reinterpret_cast<uint16_t*>(trec + cv.off_nr + 2 * slot) = valid ? f16b(sqrtf(rr[row])) : uint16_t(0);
}

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// One wave per key row: kcat row [c[idx] | +-n_r] in fp16 ([rows][d + m]),
// 8 coordinates (one byte of each bit plane) and one 16-byte store per lane
// and step; +-n_r is exact since n_r is stored as fp16.
__global__ __launch_bounds__(256) void dequant_kernel(CodecView cv, const uint8_t* rec, int64_t row0,
                                                      int64_t rows, uint16_t* kcat, float* nxv) {
  __shared__ uint16_t scen[kMaxLevels];
  if (threadIdx.x < kMaxLevels) scen[threadIdx.x] = f16b(cv.ucen[threadIdx.x]);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bool prod = cv.mode == TQ_PROD;
  const int d = cv.d, m = prod ? cv.m : 0, kw = d + m, ub = cv.ubits;
  const int64_t grow = row0 + row;
  const uint8_t* trec = rec + (grow / kTile) * cv.tile_bytes;
  const int slot = int(grow % kTile);
  uint16_t* out = kcat + row * kw;
  if (lane == 0) nxv[row] = f16v(*reinterpret_cast<const uint16_t*>(trec + cv.off_nx + 2 * slot));
  for (int c8 = lane; c8 < d / 8; c8 += 64) {
    uint32_t pb[kMaxBits];
#pragma unroll
    for (int p = 0; p < kMaxBits; ++p) {
      const int byte = p * (d / 8) + c8;
      pb[p] = p < ub ? trec[size_t(byte / 16) * kTile * 16 + size_t(slot) * 16 + byte % 16] : 0u;
    }
    u32x4v o;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 2 * k2 + h;
        int idx = 0;
#pragma unroll
        for (int p = 0; p < kMaxBits; ++p) idx |= int((pb[p] >> k) & 1u) << p;
        pair |= uint32_t(scen[idx]) << (16 * h);
      }
      o[k2] = pair;
    }
    *reinterpret_cast<u32x4v*>(out + 8 * c8) = o;
  }
  if (prod) {
    const uint32_t nr = *reinterpret_cast<const uint16_t*>(trec + cv.off_nr + 2 * slot);
    const uint32_t nn = nr ^ 0x8000u;
    for (int c8 = lane; c8 < m / 8; c8 += 64) {
      const uint32_t sb = trec[cv.off_signs + size_t(c8 / 16) * kTile * 16 + size_t(slot) * 16 + c8 % 16];
      u32x4v o;
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2)
        o[k2] = ((sb >> (2 * k2)) & 1u ? nr : nn) | (((sb >> (2 * k2 + 1)) & 1u ? nr : nn) << 16);
      *reinterpret_cast<u32x4v*>(out + d + 8 * c8) = o;
    }
  }
}

// One wave per query: row v = [q' | sqrt(pi/2)/m q_s] (d + m values), scale
// 2^e putting max |v| in [2^14, 2^15), fp16 of v 2^e as row q of out
// [nq][d + m], and inv[q] = 2^-e.
__global__ __launch_bounds__(256) void qsplit_kernel(const float* qr, const float* qs, int64_t nq,
                                                     int d, int m, float kq, uint16_t* out,
                                                     float* inv) {
  const int lane = threadIdx.x & 63;
  const int64_t q = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (q >= nq) return;
  const int w = d + m;
  auto at = [&](int i) -> float { return i < d ? qr[q * d + i] : kq * qs[q * m + (i - d)]; };
  float mx = 0.f;
  for (int i = lane; i < w; i += 64) mx = fmaxf(mx, fabsf(at(i)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const int ebits = int((__float_as_uint(mx) >> 23) & 0xff);
  const int e = mx > 0.f ? min(253, max(1, 268 - ebits)) : 127;
  const float p2 = __uint_as_float(uint32_t(e) << 23);
  for (int i = lane; i < w; i += 64) out[q * w + i] = f16b(at(i) * p2);
  if (lane == 0) inv[q] = __uint_as_float(uint32_t(254 - e) << 23);
}

// s[q][t] = nxv[t] inv[q] part[q][t]
__global__ void combine_kernel(const float* part, const float* inv, const float* nxv, int64_t nq,
                               int64_t nc, int64_t ld_parts, float* out, int64_t ld_out) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= nq * nc) return;
  const int64_t q = e / nc, t = e % nc;
  out[q * ld_out + t] = nxv[t] * (inv[q] * part[q * ld_parts + t]);
}

// ------------------------------------------------------------- rocBLAS
std::mutex g_blas_mu;
rocblas_handle g_blas[64] = {};

rocblas_handle blas(int dev) {
  if (dev < 0 || dev >= 64) return nullptr;
  if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) g_blas[dev] = nullptr;
  return g_blas[dev];
}

// Row-major C[M][N] (+)= A[M][K] * B[N][K]^T with fp16 A, B and fp32 C.
hipError_t gemm_abt(rocblas_handle h, const uint16_t* a, const uint16_t* b, float* c, int64_t M,
                    int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, bool accumulate) {
  const float one = 1.f, beta = accumulate ? 1.f : 0.f;
  // column-major: C^T (N x M) = B (N x K) * A^T, i.e. op(B_cm) = T, op(A_cm) = N
  rocblas_status st = rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none,
                                      rocblas_int(N), rocblas_int(M), rocblas_int(K), &one,
                                      b, rocblas_datatype_f16_r, rocblas_int(ldb), a,
                                      rocblas_datatype_f16_r, rocblas_int(lda), &beta, c,
                                      rocblas_datatype_f32_r, rocblas_int(ldc), c,
                                      rocblas_datatype_f32_r, rocblas_int(ldc),
                                      rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? hipSuccess : hipErrorLaunchFailure;
}

unsigned blocks_for(int64_t threads, int bs = 256) { return unsigned((threads + bs - 1) / bs); }

// Row-major C[M][N] = A[M][K] * B[N][K]^T in fp32.
hipError_t sgemm_abt(rocblas_handle h, const float* a, const float* b, float* c, int64_t M, int64_t N,
                     int64_t K) {
  const float one = 1.f, zero = 0.f;
  rocblas_status st = rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, rocblas_int(N),
                                    rocblas_int(M), rocblas_int(K), &one, b, rocblas_int(K), a,
                                    rocblas_int(K), &zero, c, rocblas_int(N));
  return st == rocblas_status_success ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace

int64_t large_encode_chunk() { return 16384; }

namespace {
struct EncodeWs {
  uint16_t *xcat, *rcat, *bpi, *bs;
  float *y, *w, *nx, *rr;
};

size_t encode_ws_layout(const CodecView& cv, void* base, EncodeWs* out) {
  const size_t C = size_t(large_encode_chunk()), d = size_t(cv.d), m = size_t(std::max(cv.m, 1));
  auto r = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t sizes[] = {r(C * 3 * d * 2), r(C * 2 * m * 2), r(d * 3 * d * 2), r(m * 2 * m * 2),
                          r(C * std::max(d, m) * 4), r(C * 4), r(C * 4), r(C * 4)};
  size_t off[8], tot = 0;
  for (int i = 0; i < 8; ++i) { off[i] = tot; tot += sizes[i]; }
  if (out) {
    uint8_t* p = static_cast<uint8_t*>(base);
    out->xcat = reinterpret_cast<uint16_t*>(p + off[0]);
    out->rcat = reinterpret_cast<uint16_t*>(p + off[1]);
    out->bpi = reinterpret_cast<uint16_t*>(p + off[2]);
    out->bs = reinterpret_cast<uint16_t*>(p + off[3]);
    out->y = reinterpret_cast<float*>(p + off[4]);
    out->w = reinterpret_cast<float*>(p + off[5]);
    out->nx = reinterpret_cast<float*>(p + off[6]);
    out->rr = reinterpret_cast<float*>(p + off[7]);
  }
  return tot;
}
}  // namespace

size_t large_encode_workspace(const CodecView& cv) { return encode_ws_layout(cv, nullptr, nullptr); }

hipError_t launch_encode_large(int device, const CodecView& cv, const EncodeArgs& a, void* ws,
                               hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  rocblas_handle h = blas(device);
  if (!h) return hipErrorLaunchFailure;
  if (rocblas_set_stream(h, s) != rocblas_status_success) return hipErrorLaunchFailure;
  const int64_t C = large_encode_chunk();
  const int d = cv.d, m = std::max(cv.m, 1);
  const bool prod = cv.mode == TQ_PROD;
  EncodeWs W;
  encode_ws_layout(cv, ws, &W);
  const int esz = a.x_bf16 ? 2 : 4;
  hipError_t e;
  if (prod) {
    hipLaunchKernelGGL(cat3_kernel, dim3(blocks_for(int64_t(m) * m)), dim3(256), 0, s, cv.sk_hi,
                       static_cast<const uint16_t*>(nullptr), int64_t(m), m, W.bs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  int cur_head = -1;
  for (int64_t b = 0; b < a.batch; ++b)
    for (int64_t hh = 0; hh < a.heads; ++hh) {
      const int hc = cv.heads > 1 ? int(hh) : 0;
      if (hc != cur_head) {  // [16 Pi_hi | 16 Pi_lo | 16 Pi_hi] of this head
        hipLaunchKernelGGL(cat3_kernel, dim3(blocks_for(int64_t(d) * d)), dim3(256), 0, s,
                           cv.rot_hi + size_t(hc) * d * d, cv.rot_lo + size_t(hc) * d * d, int64_t(d), d,
                           W.bpi);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        cur_head = hc;
      }
      const uint8_t* xs = static_cast<const uint8_t*>(a.x) + (b * a.xs_b + hh * a.xs_h) * esz;
      uint8_t* rec = a.rec + b * a.rs_b + hh * a.rs_h;
      const int64_t padded = (a.tokens + kTile - 1) / kTile * kTile;
      for (int64_t r0 = 0; r0 < padded; r0 += C) {
        const int64_t rows = std::min(C, padded - r0);
        const int64_t valid = std::max<int64_t>(0, std::min(rows, a.tokens - r0));
        if (valid > 0) {
          hipLaunchKernelGGL(rowprep_kernel, dim3(blocks_for(valid * 64)), dim3(256), 0, s,
                             xs + r0 * a.xs_t * esz, a.x_bf16, a.xs_t, valid, d, W.xcat, W.w, W.nx);
          if ((e = hipGetLastError()) != hipSuccess) return e;
          if ((e = gemm_abt(h, W.xcat, W.bpi, W.y, valid, d, 3 * d, 3 * d, 3 * d, d, false)) != hipSuccess)
            return e;
        }
        hipLaunchKernelGGL(quantize_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s, cv, W.y, W.w,
                           W.nx, r0, rows, valid, rec, W.rcat, W.rr);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (prod) {
          // z = [rh | rl] [S | S]^T  (z reuses the y buffer)
          if (valid > 0 &&
              (e = gemm_abt(h, W.rcat, W.bs, W.y, valid, m, 2 * m, 2 * m, 2 * m, m, false)) != hipSuccess)
            return e;
          hipLaunchKernelGGL(signpack_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s, cv, W.y, W.rr,
                             r0, rows, valid, rec);
          if ((e = hipGetLastError()) != hipSuccess) return e;
        }
      }
    }
  return hipSuccess;
}

// q' = Pi_head q and (prod) q_s = S q' for nq fp32 queries, as fp32 GEMMs.
hipError_t launch_query_prep_large(int device, const CodecView& cv, const float* q, int64_t nq, int head,
                                   float* qr, float* qs, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  rocblas_handle h = blas(device);
  if (!h) return hipErrorLaunchFailure;
  if (rocblas_set_stream(h, s) != rocblas_status_success) return hipErrorLaunchFailure;
  const int d = cv.d;
  const int hc = cv.heads > 1 ? head : 0;
  hipError_t e = sgemm_abt(h, q, cv.rot + size_t(hc) * d * d, qr, nq, d, d);
  if (e != hipSuccess || cv.mode != TQ_PROD) return e;
  // q_s = S q'[0:m]: rows of qr have stride d, so m must equal d here
  return sgemm_abt(h, qr, cv.sketch, qs, nq, cv.m, cv.m);
}

int64_t large_score_chunk() { return 65536; }

namespace {
struct ScoreWs {
  uint16_t *qcat, *kcat;
  float *inv, *part, *nxv;
};

size_t score_ws_layout(const CodecView& cv, int64_t nq, void* base, ScoreWs* out) {
  const size_t NC = size_t(large_score_chunk()), d = size_t(cv.d);
  const size_t kw = d + (cv.mode == TQ_PROD ? size_t(cv.m) : 0);
  auto r = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t sizes[] = {r(size_t(nq) * kw * 2), r(NC * kw * 2), r(size_t(nq) * 4),
                          r(size_t(nq) * NC * 4), r(NC * 4)};
  size_t off[5], tot = 0;
  for (int i = 0; i < 5; ++i) { off[i] = tot; tot += sizes[i]; }
  if (out) {
    uint8_t* p = static_cast<uint8_t*>(base);
    out->qcat = reinterpret_cast<uint16_t*>(p + off[0]);
    out->kcat = reinterpret_cast<uint16_t*>(p + off[1]);
    out->inv = reinterpret_cast<float*>(p + off[2]);
    out->part = reinterpret_cast<float*>(p + off[3]);
    out->nxv = reinterpret_cast<float*>(p + off[4]);
  }
  return tot;
}
}  // namespace

size_t large_score_workspace(const CodecView& cv, int64_t nq) {
  return score_ws_layout(cv, nq, nullptr, nullptr);
}

// Scores of nq prepared queries (qr [nq][d], qs [nq][m] fp32) against n
// records: s = n_x <[q' | sqrt(pi/2)/m q_s], [c[idx] | n_r sign]>, one GEMM
// per key chunk.  With out != nullptr the scores go to out[nq][n]; otherwise
// each chunk's unscaled products (row stride large_score_chunk()) and the
// scales n_x (per key) and 2^-e (per query) are handed to chunk_cb (the top-k
// search applies them as it scans).
hipError_t launch_score_large(int device, const CodecView& cv, const float* qr, const float* qs,
                              int64_t nq, const uint8_t* rec, int64_t n, float* out, void* ws,
                              hipStream_t s, ChunkFn chunk_cb, void* cb_ctx) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  rocblas_handle h = blas(device);
  if (!h) return hipErrorLaunchFailure;
  if (rocblas_set_stream(h, s) != rocblas_status_success) return hipErrorLaunchFailure;
  const int64_t NC = large_score_chunk();
  const bool prod = cv.mode == TQ_PROD;
  const int d = cv.d, m = prod ? cv.m : 0, kw = d + m;
  ScoreWs W;
  score_ws_layout(cv, nq, ws, &W);
  hipLaunchKernelGGL(qsplit_kernel, dim3(blocks_for(nq * 64)), dim3(256), 0, s, qr, qs, nq, d, m,
                     prod ? kQjl / float(cv.m) : 0.f, W.qcat, W.inv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int64_t r0 = 0; r0 < n; r0 += NC) {
    const int64_t rows = std::min(NC, n - r0);
    hipLaunchKernelGGL(dequant_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s, cv, rec, r0, rows,
                       W.kcat, W.nxv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // q kcat^T  ->  part [nq][NC]
    if ((e = gemm_abt(h, W.qcat, W.kcat, W.part, nq, rows, kw, kw, kw, NC, false)) != hipSuccess) return e;
    if (out) {
      hipLaunchKernelGGL(combine_kernel, dim3(blocks_for(nq * rows)), dim3(256), 0, s, W.part, W.inv, W.nxv,
                         nq, rows, NC, out + r0, n);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (chunk_cb && (e = chunk_cb(cb_ctx, W.part, NC, r0, rows, W.nxv, W.inv, s)) != hipSuccess) {
      return e;
    }
  }
  return hipSuccess;
}

}  // namespace tq
