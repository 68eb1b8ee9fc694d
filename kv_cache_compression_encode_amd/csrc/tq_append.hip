// Append-on-decode for d = 128: encode one new vector per (sequence, head)
// into slot `positions[b]` of that head's existing records.  TurboQuant also
// quantizes the tokens generated during decoding (TurboQuant paper review,
// "Comparison"); this writes them in place so the next decode step reads them
// like any other token.
//
// One 256-thread workgroup per vector: thread t owns coordinate i = t % 128
// over half h = t / 128 of each matrix product's reduction range.  Every
// thread issues its 64 loads of the transposed rotation (and, for a full
// sketch, of the transposed sketch) before it needs them, so the encode costs
// about one memory round trip; the two halves' sums meet in LDS.  The
// rotation and the sketch are fp32 sums (y within about 1e-7 of the exact
// rotation, far inside the 1e-5 decision band).  Codes follow the per-dim
// boundaries (ties to the upper cell), so any bit map works.  ROW records:
// the vector's bit string is assembled in LDS from the bit positions table and
// written byte by byte into its 16-byte chunks.  COL records: the thread of
// dim i rewrites the new vector's bits in dim i's field (read, mask, write; no
// other thread touches that word).  Outlier-channel split codecs: each group
// (stored coordinates i with i % 32 < o4, and the rest) is normalised by its
// own norm, taken from its rotated coordinates (the rotation is orthogonal on
// each group's channels), and keeps its own n_x and n_r.
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

// Sum over the 128 coordinates (threads 0..127, waves 0 and 1) of two values;
// every thread gets both sums.  red: 4 floats of LDS.
__device__ __forceinline__ void coord_sums(float a, float b, float* red, float& sa, float& sb) {
  const int t = threadIdx.x, w = t >> 6;
  a = wave_sum(t < D ? a : 0.f);
  b = wave_sum(t < D ? b : 0.f);
  if ((t & 63) == 0 && w < 2) {
    red[w] = a;
    red[2 + w] = b;
  }
  __syncthreads();
  sa = red[0] + red[1];
  sb = red[2] + red[3];
  __syncthreads();
}

// One vector of one codec; `append_kernel` and `append_pair_kernel` (the key
// and the value of a decode step in one launch) call it per workgroup.
__device__ __forceinline__ void append_one(const CodecView& cv, const AppendArgs& a, int hd, int b) {
  const int t = threadIdx.x;
  const int i = t & (D - 1), half = t >> 7;
  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.capacity) return;  // outside the cache: nothing written
  const int hc = cv.heads > 1 ? hd : 0;
  const int m = cv.mode == TQ_PROD ? cv.m : 0;
  const bool full_sketch = m == D;
  __shared__ float sx[D], sr[D], part[2][D], red[4];
  __shared__ uint32_t sbits[5 * D / 32 + 4], ssign[D / 32];

  // ---- tables first: they do not depend on the vector.  Matrix columns
  // (all threads), and for dim i (threads < 128) its bit count, boundaries,
  // levels and bit positions.
  float rcol[D / 2], scol[D / 2], thr[kMaxLevels - 1], cen[kMaxLevels];
  int nbits = 0;
  int bpos[kMaxBits];
  if (t < D) {
    nbits = cv.dim_bits[i];
    const float* tt = cv.thr + (size_t(hc) * D + i) * kMaxLevels;
    const float* cc = cv.cen + (size_t(hc) * D + i) * kMaxLevels;
#pragma unroll
    for (int k = 0; k < kMaxLevels - 1; ++k) thr[k] = tt[k];
#pragma unroll
    for (int k = 0; k < kMaxLevels; ++k) cen[k] = cc[k];
#pragma unroll
    for (int p = 0; p < kMaxBits; ++p) bpos[p] = cv.bitpos[p * D + i];
  }
  // randomized Hadamard rotation: z = H (s x) / sqrt(d) by the wave
  // transform instead of the columns of Pi
  const bool had = cv.had_sign != nullptr;
  {
    const float* rt = cv.rot_t + size_t(hc) * D * D + size_t(64 * half) * D + i;
    if (!had) {
#pragma unroll
      for (int u = 0; u < D / 2; ++u) rcol[u] = rt[size_t(u) * D];
    }
    if (full_sketch) {
      const float* st = cv.sketch_t + size_t(64 * half) * D + i;
#pragma unroll
      for (int u = 0; u < D / 2; ++u) scol[u] = st[size_t(u) * D];
    }
  }
  // ---- the vector
  const int64_t xo = int64_t(b) * a.xs_b + int64_t(hd) * a.xs_h;
  if (t < D) {
    sx[t] = a.x_bf16 ? __uint_as_float(uint32_t(static_cast<const uint16_t*>(a.x)[xo + t]) << 16)
                     : static_cast<const float*>(a.x)[xo + t];
  }
  if (t < int(sizeof(sbits) / 4)) sbits[t] = 0u;
  if (t < D / 32) ssign[t] = 0u;
  __syncthreads();

  // ---- z = Pi x (unnormalised): half sums, then coordinate i on threads < 128
  if (had) {
    // wave 0 transforms, wave 1 zeroes the second half's sums
    const int lane = t & 63, wv = t >> 6;
    if (wv == 0) {
      float lo = sx[lane] * cv.had_sign[lane], hi = sx[lane + 64] * cv.had_sign[lane + 64];
      fwht128_wave(lo, hi, lane);
      part[0][lane] = lo * kInvSqrt128;
      part[0][lane + 64] = hi * kInvSqrt128;
    } else if (wv == 1) {
      part[1][lane] = 0.f;
      part[1][lane + 64] = 0.f;
    }
  } else {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int u = 0; u < D / 2; u += 2) {
      s0 = fmaf(rcol[u], sx[64 * half + u], s0);
      s1 = fmaf(rcol[u + 1], sx[64 * half + u + 1], s1);
    }
    part[half][i] = s0 + s1;
  }
  __syncthreads();
  const float z = part[0][i] + part[1][i];
  // norms: ||x|| (all coordinates), or per group for a split codec
  const bool og = cv.outl && (i & 31) < cv.o4;
  float nxo = 0.f, nxr = 0.f;
  {
    const float xv = t < D ? sx[t] : 0.f;
    const float q = cv.outl ? z * z : xv * xv;
    coord_sums(og ? q : 0.f, og ? 0.f : q, red, nxo, nxr);
    if ((cv.outl && nxo < 0x1p-100f) || nxr < 0x1p-100f) {
      // a norm below 2^-50 (squares that may be denormal or flushed) or a
      // zero group: the sums again over the values times 2^64 (exact
      // scaling); the sums are the same on every thread, so is the branch
      const float zs = z * 0x1p64f, xs = xv * 0x1p64f;
      const float q2 = cv.outl ? zs * zs : xs * xs;
      coord_sums(og ? q2 : 0.f, og ? 0.f : q2, red, nxo, nxr);
      nxo = sqrtf(nxo) * 0x1p-64f;
      nxr = sqrtf(nxr) * 0x1p-64f;
    } else {
      nxo = sqrtf(nxo);
      nxr = sqrtf(nxr);
    }
  }
  const float ng = og ? nxo : nxr;
  const float inv = ng > 0.f ? 1.f / ng : 0.f;  // a zero vector (group) encodes y = 0
  const float y = z * inv;

  // ---- quantize dim i: idx = number of boundaries <= y
  int idx = 0;
  float res = 0.f;
  if (t < D) {
    const int L = 1 << nbits;
#pragma unroll
    for (int k = 0; k < kMaxLevels - 1; ++k)
      if (k < L - 1) idx += thr[k] <= y ? 1 : 0;
    float c = cen[0];  // cen[idx], by selects (no indexed register array)
#pragma unroll
    for (int k = 1; k < kMaxLevels; ++k) c = idx == k ? cen[k] : c;
    res = i < m ? y - c : 0.f;
  }
  const int slot = pos % kTile, tile = pos / kTile;
  uint8_t* trec;
  if (a.block_table) {
    trec = a.rec + paged_tile(a.block_table, a.page_shift, a.max_pages, int64_t(b) * a.H + hd, tile) * cv.tile_bytes;
  } else {
    trec = a.rec + int64_t(b) * a.rs_b + int64_t(hd) * a.rs_h + int64_t(tile) * cv.tile_bytes;
  }

  // ---- codes
  if (cv.layout == TQ_LAYOUT_ROW) {
    if (t < D)
#pragma unroll
      for (int p = 0; p < kMaxBits; ++p)
        if (p < nbits && ((idx >> p) & 1)) {
          const int P = bpos[p];
          atomicOr(&sbits[P >> 5], 1u << (P & 31));
        }
  } else if (t < D && cv.outl) {
    // col records of the 2.5-bit split: bits b k .. b k + b - 1 of
    // coordinate i's b-byte word in the slot's 8-token group (k = slot % 8),
    // the word at byte 5 (vb / 2) + 3 (vb % 2) of lane block n < 8 (20 bytes)
    // or 2 vb of block n >= 8 (16 bytes; n = i % 16, vb = i / 16), 288 bytes a
    // group; the other tokens' bits are kept
    const int n = i & 15, vb = i >> 4;
    const int off = n < 8 ? 20 * n + 5 * (vb >> 1) + 3 * (vb & 1) : 160 + 16 * (n - 8) + 2 * vb;
    uint8_t* wb = trec + (slot >> 3) * 288 + off;
    const int ub = nbits, sh = ub * (slot & 7);
    uint32_t w = 0u;
    for (int q = 0; q < ub; ++q) w |= uint32_t(wb[q]) << (8 * q);
    const uint32_t mask = ((1u << ub) - 1u) << sh;
    w = (w & ~mask) | ((uint32_t(idx) << sh) & mask);
    for (int q = 0; q < ub; ++q) wb[q] = uint8_t(w >> (8 * q));
  } else if (t < D) {
    // col: bit (b v + k) of dim i's 8b-byte field is bit k of vector v's index
    const int ub = nbits;  // uniform codec: the same on every dim
    uint32_t* wp = reinterpret_cast<uint32_t*>(trec + size_t(i) * 8 * ub) + (ub * slot) / 32;
    const int sh = (ub * slot) % 32;
    const uint32_t mask = ((1u << ub) - 1u) << sh;
    *wp = (*wp & ~mask) | ((uint32_t(idx) << sh) & mask);
  }

  // ---- prod: residual norms and the QJL sketch signs
  float nr = 0.f, nro = 0.f;
  if (cv.mode == TQ_PROD) {
    if (t < D) sr[t] = res;
    const float rq = res * res;
    coord_sums(og ? rq : 0.f, og ? 0.f : rq, red, nro, nr);  // also orders the sr writes
    nr = sqrtf(nr);
    nro = sqrtf(nro);
    if (full_sketch) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int u = 0; u < D / 2; u += 2) {
        s0 = fmaf(scol[u], sr[64 * half + u], s0);
        s1 = fmaf(scol[u + 1], sr[64 * half + u + 1], s1);
      }
      part[half][i] = s0 + s1;
      __syncthreads();
      if (t < D && part[0][t] + part[1][t] >= 0.f) atomicOr(&ssign[t >> 5], 1u << (t & 31));  // sign(0) = +1
    } else if (t < m) {
      float zz = 0.f;
      for (int k = 0; k < m; ++k) zz = fmaf(cv.sketch_t[size_t(k) * m + t], sr[k], zz);
      if (zz >= 0.f) atomicOr(&ssign[t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
  if (cv.layout == TQ_LAYOUT_ROW)
    for (int B_ = t; B_ < cv.code_bytes; B_ += blockDim.x) {  // byte B_ of the bit string
      const int c = B_ / 16, w = min(16, cv.code_bytes - 16 * c);
      trec[size_t(c) * kTile * 16 + size_t(slot) * w + (B_ % 16)] = uint8_t(sbits[B_ >> 2] >> (8 * (B_ & 3)));
    }
  if (cv.mode == TQ_PROD) {
    for (int B_ = t; B_ < cv.sign_bytes; B_ += blockDim.x) {
      const int c = B_ / 16, w = min(16, cv.sign_bytes - 16 * c);
      trec[cv.off_signs + size_t(c) * kTile * 16 + size_t(slot) * w + (B_ % 16)] =
          uint8_t(ssign[B_ >> 2] >> (8 * (B_ & 3)));
    }
    if (t == 0) *reinterpret_cast<uint16_t*>(trec + cv.off_nr + 2 * slot) = f16_bits(nr);
    if (t == 0 && cv.outl) *reinterpret_cast<uint16_t*>(trec + cv.off_nro + 2 * slot) = f16_bits(nro);
  }
  if (t == 0) *reinterpret_cast<uint16_t*>(trec + cv.off_nx + 2 * slot) = f16_bits(nxr);
  if (t == 0 && cv.outl) *reinterpret_cast<uint16_t*>(trec + cv.off_nxo + 2 * slot) = f16_bits(nxo);
}

__global__ __launch_bounds__(256) void append_kernel(CodecView cv, AppendArgs a) {
  append_one(cv, a, blockIdx.x, blockIdx.y);
}

// blockIdx.z = 0: the key codec and arguments, 1: the value ones
__global__ __launch_bounds__(256) void append_pair_kernel(CodecView kc, AppendArgs ka, CodecView vc,
                                                          AppendArgs va) {
  if (blockIdx.z == 0)
    append_one(kc, ka, blockIdx.x, blockIdx.y);
  else
    append_one(vc, va, blockIdx.x, blockIdx.y);
}

}  // namespace

bool append_supported(const CodecView& cv) {
  if (cv.d != D || !cv.rot_t) return false;
  if (cv.layout == TQ_LAYOUT_COL) {
    if (cv.outl) return cv.mode == TQ_MSE && cv.o4 == 8 && cv.split_ub_o == 3 && cv.split_ub_r == 2;
    return cv.uniform && cv.mode == TQ_MSE && (cv.ubits == 1 || cv.ubits == 2 || cv.ubits == 4);
  }
  return cv.mode == TQ_MSE || (cv.sketch_t && cv.m >= 1 && cv.m <= D);
}

hipError_t launch_append(const CodecView& cv, const AppendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(unsigned(a.H), unsigned(a.B)), dim3(256), 0, s, cv, a);
  return hipGetLastError();
}

hipError_t launch_append_pair(const CodecView& kc, const AppendArgs& ka, const CodecView& vc,
                              const AppendArgs& va, hipStream_t s) {
  if (ka.H != va.H || ka.B != va.B) return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_pair_kernel, dim3(unsigned(ka.H), unsigned(ka.B), 2u), dim3(256), 0, s, kc, ka,
                     vc, va);
  return hipGetLastError();
}

}  // namespace tq
