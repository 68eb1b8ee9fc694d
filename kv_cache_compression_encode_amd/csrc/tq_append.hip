// Append-on-decode for d = 128: encode one new vector per (sequence, head)
// into slot `positions[b]` of that head's existing records.  TurboQuant also
// quantizes the tokens generated during decoding (TurboQuant paper review,
// "Comparison"); this writes them in place so the next decode step reads them
// like any other token.
//
// One wavefront per vector, lane l owning dims l and l + 64.  The rotation and
// the sketch run in fp32 on the VALU through the transposed matrices
// (column-coalesced loads); fp32 sums of 128 terms put y within about 1e-7
// of the exact rotation, far inside the 1e-5 decision band.  Codes follow the
// per-dim boundaries (ties to the upper cell), so any bit map works.  ROW
// records: the vector's bit string is assembled in LDS from the bit positions
// table and written byte by byte into its 16-byte chunks.  COL records: each
// lane rewrites the bits of its two dims in the dims' fields (read, mask,
// write; no other wave touches these words).  Outlier-channel split codecs:
// each group (stored coordinates i with i % 32 < o4, and the rest) is
// normalised by its own norm, taken from its rotated coordinates (the
// rotation is orthogonal on each group's channels), and keeps its own n_x and
// n_r.
#include <hip/hip_runtime.h>

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int D = 128;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint16_t f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

__global__ __launch_bounds__(64) void append_kernel(CodecView cv, AppendArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, l = threadIdx.x;
  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.capacity) return;  // outside the cache: nothing written
  const int hc = cv.heads > 1 ? h : 0;
  __shared__ float sx[D], sr[D];
  __shared__ uint32_t sbits[5 * D / 32 + 4], ssign[D / 32];

  // ---- input and norm
  const int64_t xo = int64_t(b) * a.xs_b + int64_t(h) * a.xs_h;
  float x0, x1;
  if (a.x_bf16) {
    const uint16_t* xp = static_cast<const uint16_t*>(a.x) + xo;
    x0 = __uint_as_float(uint32_t(xp[l]) << 16);
    x1 = __uint_as_float(uint32_t(xp[l + 64]) << 16);
  } else {
    const float* xp = static_cast<const float*>(a.x) + xo;
    x0 = xp[l];
    x1 = xp[l + 64];
  }
  const float nx = sqrtf(wave_sum(fmaf(x0, x0, x1 * x1)));
  float inv = nx > 0.f ? 1.f / nx : 0.f;  // a zero vector encodes y = 0
  sx[l] = x0;
  sx[l + 64] = x1;
  if (l < int(sizeof(sbits) / 4)) sbits[l] = 0u;
  if (l < D / 32) ssign[l] = 0u;
  __syncthreads();

  // ---- y = Pi x / ||x||, dims l and l + 64
  const float* rt = cv.rot_t + size_t(hc) * D * D;
  float a0 = 0.f, a1 = 0.f, c0 = 0.f, c1 = 0.f;
#pragma unroll 8
  for (int k = 0; k < D; k += 2) {
    a0 = fmaf(rt[size_t(k) * D + l], sx[k], a0);
    a1 = fmaf(rt[size_t(k) * D + l + 64], sx[k], a1);
    c0 = fmaf(rt[size_t(k + 1) * D + l], sx[k + 1], c0);
    c1 = fmaf(rt[size_t(k + 1) * D + l + 64], sx[k + 1], c1);
  }
  const float z0 = a0 + c0, z1 = a1 + c1;
  // split: lane l's dims l and l + 64 share l % 32, so one group per lane
  const bool og = cv.outl && (l & 31) < cv.o4;
  float nxo = 0.f, nxr = nx;
  if (cv.outl) {
    const float q = fmaf(z0, z0, z1 * z1);
    nxo = sqrtf(wave_sum(og ? q : 0.f));
    nxr = sqrtf(wave_sum(og ? 0.f : q));
    const float ng = og ? nxo : nxr;
    inv = ng > 0.f ? 1.f / ng : 0.f;
  }
  const float y[2] = {z0 * inv, z1 * inv};

  // ---- quantize: idx = number of boundaries <= y
  int idx[2];
  float res[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = l + 64 * u;
    const int L = 1 << cv.dim_bits[i];
    const float* t = cv.thr + (size_t(hc) * D + i) * kMaxLevels;
    int k = 0;
    for (int q = 0; q < L - 1; ++q) k += t[q] <= y[u] ? 1 : 0;
    idx[u] = k;
    res[u] = i < cv.m ? y[u] - cv.cen[(size_t(hc) * D + i) * kMaxLevels + k] : 0.f;
  }
  const int slot = pos % kTile, tile = pos / kTile;
  uint8_t* trec;
  if (a.block_table) {
    trec = a.rec + paged_tile(a.block_table, a.page_shift, a.max_pages, int64_t(b) * a.H + h, tile) * cv.tile_bytes;
  } else {
    trec = a.rec + int64_t(b) * a.rs_b + int64_t(h) * a.rs_h + int64_t(tile) * cv.tile_bytes;
  }

  // ---- codes
  if (cv.layout == TQ_LAYOUT_ROW) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = l + 64 * u;
      for (int p = 0; p < cv.dim_bits[i]; ++p)
        if ((idx[u] >> p) & 1) {
          const int P = cv.bitpos[p * D + i];
          atomicOr(&sbits[P >> 5], 1u << (P & 31));
        }
    }
    __syncthreads();
    for (int B = l; B < cv.code_bytes; B += 64) {  // byte B of the bit string
      const int c = B / 16, w = min(16, cv.code_bytes - 16 * c);
      trec[size_t(c) * kTile * 16 + size_t(slot) * w + (B % 16)] = uint8_t(sbits[B >> 2] >> (8 * (B & 3)));
    }
  } else {
    // col: bit (b v + k) of dim i's 8b-byte field is bit k of vector v's index
    const int ub = cv.dim_bits[0];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = l + 64 * u;
      uint32_t* wp = reinterpret_cast<uint32_t*>(trec + size_t(i) * 8 * ub) + (ub * slot) / 32;
      const int sh = (ub * slot) % 32;
      const uint32_t mask = ((1u << ub) - 1u) << sh;
      *wp = (*wp & ~mask) | ((uint32_t(idx[u]) << sh) & mask);
    }
  }

  // ---- prod: residual norm and the QJL sketch signs
  if (cv.mode == TQ_PROD) {
    const float rq = fmaf(res[0], res[0], res[1] * res[1]);
    const float nr = sqrtf(wave_sum(og ? 0.f : rq));
    const float nro = cv.outl ? sqrtf(wave_sum(og ? rq : 0.f)) : 0.f;
    sr[l] = res[0];
    sr[l + 64] = res[1];
    __syncthreads();
    const int m = cv.m;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = l + 64 * u;
      if (j < m) {
        float z = 0.f, z2 = 0.f;
        int i = 0;
        for (; i + 1 < m; i += 2) {
          z = fmaf(cv.sketch_t[size_t(i) * m + j], sr[i], z);
          z2 = fmaf(cv.sketch_t[size_t(i + 1) * m + j], sr[i + 1], z2);
        }
        if (i < m) z = fmaf(cv.sketch_t[size_t(i) * m + j], sr[i], z);
        if (z + z2 >= 0.f) atomicOr(&ssign[j >> 5], 1u << (j & 31));  // sign(0) = +1
      }
    }
    __syncthreads();
    for (int B = l; B < cv.sign_bytes; B += 64) {
      const int c = B / 16, w = min(16, cv.sign_bytes - 16 * c);
      trec[cv.off_signs + size_t(c) * kTile * 16 + size_t(slot) * w + (B % 16)] =
          uint8_t(ssign[B >> 2] >> (8 * (B & 3)));
    }
    if (l == 0) *reinterpret_cast<uint16_t*>(trec + cv.off_nr + 2 * slot) = f16_bits(nr);
    if (l == 0 && cv.outl) *reinterpret_cast<uint16_t*>(trec + cv.off_nro + 2 * slot) = f16_bits(nro);
  }
  if (l == 0) *reinterpret_cast<uint16_t*>(trec + cv.off_nx + 2 * slot) = f16_bits(nxr);
  if (l == 0 && cv.outl) *reinterpret_cast<uint16_t*>(trec + cv.off_nxo + 2 * slot) = f16_bits(nxo);
}

}  // namespace

bool append_supported(const CodecView& cv) {
  if (cv.d != D || !cv.rot_t) return false;
  if (cv.layout == TQ_LAYOUT_COL)
    return cv.uniform && cv.mode == TQ_MSE && (cv.ubits == 1 || cv.ubits == 2 || cv.ubits == 4);
  return cv.mode == TQ_MSE || (cv.sketch_t && cv.m >= 1 && cv.m <= D);
}

hipError_t launch_append(const CodecView& cv, const AppendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(unsigned(a.H), unsigned(a.B)), dim3(64), 0, s, cv, a);
  return hipGetLastError();
}

}  // namespace tq
