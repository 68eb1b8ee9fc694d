// Internal declarations shared by the host builder, the C-ABI layer and the
// HIP kernels of the codec library.  Not part of the public ABI.
#pragma once

#include <cstdint>
#include <vector>

#include "tq.h"

namespace tq {

constexpr int kTile = TQ_TILE;
constexpr int kMaxLevels = TQ_MAX_LEVELS;
constexpr int kMaxBits = TQ_MAX_BITS;

// ---------------------------------------------------------------- host math
// Philox4x32-10 (Salmon et al., SC'11) and Box-Muller normals.
void philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
void philox_normals(uint64_t seed, uint32_t stream, int64_t count, double* out);

// Householder QR of a square matrix g (row-major n x n); returns
// Pi = Q diag(sign(R_ii)) row-major.
void haar_from_gaussian(int n, const double* g, double* pi);

// Lloyd-Max solution of a symmetric scalar law.
struct LloydMaxResult {
  std::vector<double> centroids, boundaries;
  double mse = 0;
  int iterations = 0;
};
// Law of one coordinate of a uniformly random unit vector in R^d.
LloydMaxResult lloyd_max_sphere(int d, int bits);
// Standard normal law.
LloydMaxResult lloyd_max_gaussian(int bits);

// Symmetric eigendecomposition (cyclic Jacobi).  a: n x n row-major symmetric.
// Returns eigenvalues descending and eigenvectors as rows (row i <-> lambda_i),
// each row signed so that its largest-magnitude entry (first on ties) is > 0.
void symmetric_eigen(int n, const double* a, double* lambda, double* rows);

// tq_decode_attend with the caller's workspace (shared by the allocating and
// the allocation-free entry points).
tq_status decode_attend_ws(const tq_codebook* kcb, const tq_codebook* vcb, const void* q, int32_t q_dtype,
                           int32_t B, int32_t Hq, int32_t Hkv, const tq_kv_view* kv, float softmax_scale,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

uint16_t f32_to_bf16_rne(float x);
float bf16_to_f32(uint16_t h);
uint16_t f32_to_f16_rne(float x);
float f16_to_f32(uint16_t h);

// --------------------------------------------------------- kernel parameters
// Device tables of a codebook.
struct DeviceTables {
  float* rot = nullptr;          // [H][d][d] fp32, row i = basis vector i
  float* rot_t = nullptr;        // [H][d][d] fp32 transpose (column-coalesced reads)
  uint16_t* rot_hi = nullptr;    // [H][d][d] fp16 high part of 16 Pi
  uint16_t* rot_lo = nullptr;    // [H][d][d] fp16 residual part of 16 Pi
  float* sketch = nullptr;       // [m][m] fp32
  float* sketch_t = nullptr;     // [m][m] fp32 transpose
  uint16_t* sketch_hi = nullptr; // [m][m] fp16 high part
  uint16_t* sketch_lo = nullptr; // [m][m] fp16 residual part
  float* thr = nullptr;          // [H][d][kMaxLevels] boundaries (unused = +inf)
  float* cen = nullptr;          // [H][d][kMaxLevels] centroids
  int16_t* bitpos = nullptr;     // [kMaxBits][d] bit position in the ROW bit string, -1 if absent
  uint8_t* dim_bits = nullptr;   // [d]
  // non-uniform d = 128 codecs: decode tables of the one-bit dims and the
  // tail byte (built once here instead of in every decode workgroup)
  uint32_t* sq_tail = nullptr;   // [256] tail byte -> index bits 1.. of dims 0..3, 5 bits per dim
  float* sq_gm = nullptr;        // [H][2][d] (c1 - c0) / 2 and (c1 + c0) / 2 per dim
  // randomized Hadamard rotation at d = 128: per half h of the input (dims
  // 64h .. 64h + 63) and packed bf16 pair k, the sign bits (15 and 31) to flip
  uint32_t* had_mask = nullptr;  // [2][32]
  float* had_sign = nullptr;     // [d] the signs s as +-1.0f (query and value-output transforms)
  // outlier-channel split: per head, bit c of the 128-bit mask = channel c is an outlier
  uint32_t* omask = nullptr;     // [H][4]
  // wide uniform codecs (d a multiple of 128 other than 128): the rotation and
  // sketch in the tile order of the MFMA kernels, rows of each 32-row group
  // permuted so that a half-wave's accumulators hold 16 consecutive rows
  uint16_t* rot_tiles = nullptr; // [d/128][d/32][2][128][32] fp16 hi, lo of 16 Pi
  uint16_t* sk_tiles = nullptr;  // [m/128][m/32][128][32] fp16 S
};

}  // namespace tq

struct tq_codebook {
  tq_codebook_desc desc{};
  tq_codebook_info info{};
  int device = 0;
  int m = 0;
  bool uniform = true;
  int ubits = 0;  // index bits when uniform
  int outlier = 0;  // o of an outlier-channel split codec (stored order), else 0
  std::vector<uint32_t> omask;  // split: [H][d / 32] outlier-channel bit masks
  std::vector<uint8_t> bits;                 // [d]
  std::vector<double> rot64;                 // [H][d][d] (fp64 before rounding)
  std::vector<float> rot32;                  // [H][d][d]
  std::vector<float> sketch32;               // [m][m]
  std::vector<double> cen64, thr64;          // [H][d][kMaxLevels], [H][d][kMaxLevels-1]
  std::vector<float> cen32, thr32;           // [H][d][kMaxLevels]
  std::vector<int16_t> bitpos;               // [kMaxBits][d]
  std::vector<int8_t> hsign;                 // TQ_ROT_HADAMARD: the signs s [d]
  tq::DeviceTables dev;
};
