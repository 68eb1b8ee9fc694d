// Query preparation, compressed-key scoring, fused decode attention and top-k
// search over TurboQuant records (gfx950).
//
// Scoring follows the TurboQuant paper review ("Method"): with q' = Pi q and
// qs = S q'[0:m], a record (idx, signs, n_x, n_r) scores
//   s = n_x ( sum_i q'_i c_i[idx_i] + n_r sqrt(pi/2)/m sum_j qs_j (2 bit_j - 1) ).
// Decode attention applies softmax(scale * s) over the tokens of a KV head
// and accumulates p * n_v * c_v[idx_v] in the rotated value domain; the single
// inverse rotation Pi_v^T is applied once per query head after the split-K
// merge (rotation and codebook lookup fused into attention: paper review,
// "Sparks").
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kQjl = 1.2533141373155001f;  // sqrt(pi / 2)

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return float(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ----------------------------------------------------------- query prep
// Block: qb (<= 8) consecutive queries of one rotation head, staged in LDS.
// Thread t computes output coordinate t % 128 over the half t / 128 of the
// reduction range, reading the transposed matrices column-coalesced.  All
// matrix loads (Pi and, for the full sketch, S) are issued before anything
// waits, so the kernel costs about one memory round trip; the two halves'
// partial sums meet in LDS.  d = 128.
__global__ __launch_bounds__(256) void query_prep_kernel(CodecView cv, QueryPrepArgs a, int qb) {
  constexpr int D = 128, KH = 64;
  extern __shared__ float sq[];  // [qb][D] input | [qb][D] rotated | [2][qb][D] partials
  float* sr = sq + qb * D;
  float* sp = sr + qb * D;
  const int64_t q0 = int64_t(blockIdx.x) * qb;
  const int nqb = int(min<int64_t>(qb, a.nq - q0));
  int head = a.fixed_head;
  if (a.q_per_head > 0) head = int((q0 / a.q_per_head) % a.hkv);
  if (cv.heads == 1) head = 0;
  const int i = threadIdx.x & (D - 1), kh = threadIdx.x >> 7;
  const bool full_sketch = cv.mode == TQ_PROD && cv.m == D;
  const float* rt = cv.rot_t + size_t(head) * D * D + size_t(KH * kh) * D + i;
  const float* st = cv.sketch_t + size_t(KH * kh) * D + i;
  // randomized Hadamard rotation: q' = H (s q) / sqrt(d) by the wave
  // transform, so no columns of Pi are read
  const bool had = cv.had_sign != nullptr;
  float r[KH], sk[KH];
  if (!had) {
#pragma unroll
    for (int u = 0; u < KH; ++u) r[u] = rt[size_t(u) * D];
  }
  if (full_sketch) {
#pragma unroll
    for (int u = 0; u < KH; ++u) sk[u] = st[size_t(u) * D];
  }
  for (int e = threadIdx.x; e < nqb * D; e += blockDim.x) {
    const int64_t qi = q0 + e / D;
    const int c = e % D;
    float v;
    if (a.q_bf16)
      v = __uint_as_float(uint32_t(static_cast<const uint16_t*>(a.q)[qi * D + c]) << 16);
    else
      v = static_cast<const float*>(a.q)[qi * D + c];
    sq[e] = v;
  }
  __syncthreads();
  auto matvec = [&](const float (&m)[KH], const float* src, float* dst, float* gdst, int gld) {
    for (int qq = 0; qq < nqb; ++qq) {
      const float* x = src + qq * D + KH * kh;
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int u = 0; u < KH; u += 2) {
        acc0 = fmaf(m[u], x[u], acc0);
        acc1 = fmaf(m[u + 1], x[u + 1], acc1);
      }
      sp[(kh * qb + qq) * D + i] = acc0 + acc1;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nqb * D; e += blockDim.x) {
      const int qq = e / D, c = e % D;
      const float v = sp[qq * D + c] + sp[(qb + qq) * D + c];
      if (dst) dst[qq * D + c] = v;
      gdst[(q0 + qq) * gld + c] = v;
    }
    __syncthreads();
  };
  if (had) {
    const int lane = threadIdx.x & 63;
    const float s_lo = cv.had_sign[lane], s_hi = cv.had_sign[lane + 64];
    for (int qq = threadIdx.x >> 6; qq < nqb; qq += blockDim.x >> 6) {  // one query per wave
      float lo = sq[qq * D + lane] * s_lo, hi = sq[qq * D + lane + 64] * s_hi;
      fwht128_wave(lo, hi, lane);
      lo *= kInvSqrt128;
      hi *= kInvSqrt128;
      sr[qq * D + lane] = lo;
      sr[qq * D + lane + 64] = hi;
      a.qr[(q0 + qq) * D + lane] = lo;
      a.qr[(q0 + qq) * D + lane + 64] = hi;
    }
    __syncthreads();
  } else {
    matvec(r, sq, sr, a.qr, D);
  }
  if (cv.mode != TQ_PROD) return;
  if (full_sketch) {
    matvec(sk, sr, nullptr, a.qs, D);
  } else {
    for (int e = threadIdx.x; e < nqb * cv.m; e += blockDim.x) {
      const int qq = e / cv.m, j = e % cv.m;
      float acc = 0.f;
      for (int k = 0; k < cv.m; ++k) acc = fmaf(cv.sketch[size_t(j) * cv.m + k], sr[qq * D + k], acc);
      a.qs[(q0 + qq) * cv.m + j] = acc;
    }
  }
}

// Index of dim `dim` of the vector in the 16-byte code chunks of a ROW
// record (uniform codec: plane p occupies bits [p*d, (p+1)*d)).
__device__ __forceinline__ int row_index_uniform(const uint8_t* tile, int slot, int dim, int d,
                                                 int ubits) {
  int idx = 0;
  for (int p = 0; p < ubits; ++p) {
    const int bitpos = p * d + dim;
    const int chunk = bitpos >> 7, inchunk = bitpos & 127;
    const uint8_t byte = tile[size_t(chunk) * kTile * 16 + size_t(slot) * 16 + (inchunk >> 3)];
    idx |= ((byte >> (inchunk & 7)) & 1) << p;
  }
  return idx;
}

// Bit P of a vector's ROW bit string: chunk P / 128 of the tile is stored
// [64 vectors][w] with w = 16 except for a shorter last chunk.
__device__ __forceinline__ int row_bit(const uint8_t* tile, int slot, int P, int code_bytes) {
  const int c = P >> 7, w = min(16, code_bytes - 16 * c);
  return (tile[size_t(c) * kTile * 16 + size_t(slot) * w + ((P & 127) >> 3)] >> (P & 7)) & 1;
}

// ------------------------------------------------------------------ score
// d = 128.  Block = 4 waves, each wave one record tile (lane = vector); QB
// queries per block.  A lane loads its vector's record rows with 16-byte
// loads (the bit planes, the sign row) and walks the coordinates on
// registers; the queries sit in LDS as [coordinate][QB] so one 16-byte LDS
// read serves the QB products of a coordinate.
template <int QB>
__global__ __launch_bounds__(256) void score_kernel(CodecView cv, const float* qr, const float* qs,
                                                    int64_t nq, const uint8_t* rec, int64_t n,
                                                    float* scores, int head) {
  static_assert(QB == 4, "four queries per block");
  constexpr int D = 128;
  __shared__ float4 sqr[D];        // [coordinate] -> QB queries
  __shared__ float4 sqs[D];        // [sketch row] -> QB queries
  __shared__ float scen[D * kMaxLevels];
  __shared__ int16_t sbp[kMaxBits * D];  // split codecs: bit positions of the index bits
  const int m = cv.m;
  const int64_t q0 = int64_t(blockIdx.y) * QB;
  const int nqb = int(min<int64_t>(QB, nq - q0));
  for (int e = threadIdx.x; e < D * QB; e += blockDim.x) {
    const int i = e / QB, qq = e % QB;
    reinterpret_cast<float*>(sqr)[e] = qq < nqb ? qr[(q0 + qq) * D + i] : 0.f;
    reinterpret_cast<float*>(sqs)[e] = (qq < nqb && i < m) ? qs[(q0 + qq) * m + i] : 0.f;
  }
  const int ncen = cv.uniform ? kMaxLevels : D * kMaxLevels;
  const float* hcen = cv.cen + size_t(head) * D * kMaxLevels;  // the head's per-dim levels
  for (int e = threadIdx.x; e < ncen; e += blockDim.x) scen[e] = cv.uniform ? cv.ucen[e] : hcen[e];
  if (cv.outl)
    for (int e = threadIdx.x; e < kMaxBits * D; e += blockDim.x) sbp[e] = cv.bitpos[e];
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tile = int64_t(blockIdx.x) * 4 + wave;
  if (tile * kTile >= n) return;
  const int64_t v = tile * kTile + lane;
  const uint8_t* trec = rec + tile * cv.tile_bytes;
  // record rows of this lane's vector
  const int np = cv.uniform ? cv.ubits : 1;
  u32x4 pl[kMaxBits];
#pragma unroll
  for (int p = 0; p < kMaxBits; ++p)
    pl[p] = p < np ? *reinterpret_cast<const u32x4*>(trec + size_t(p) * kTile * 16 + size_t(lane) * 16)
                   : u32x4{0, 0, 0, 0};
  uint32_t tail = 0;
  if (!cv.uniform) {
    const int tb = cv.code_bytes - 16;  // 1..4 tail bytes
    for (int k = 0; k < tb; ++k) tail |= uint32_t(trec[size_t(kTile) * 16 + size_t(lane) * tb + k]) << (8 * k);
  }
  if (cv.outl) {
    // outlier-channel split: stored coordinate 32 w + k belongs to the
    // outlier instance for k < o4; each group has its own norms and QJL
    // factor sqrt(pi/2) / m_g, m_g = the group's size
    float4 ao = make_float4(0.f, 0.f, 0.f, 0.f), ar = ao, so = ao, sr = ao;
    const u32x4 sg = cv.mode == TQ_PROD ? *reinterpret_cast<const u32x4*>(trec + cv.off_signs + size_t(lane) * 16)
                                        : u32x4{0, 0, 0, 0};
    for (int w = 0; w < 4; ++w) {
#pragma unroll 4
      for (int k = 0; k < 32; ++k) {
        const int dim = 32 * w + k;
        int idx = int((pl[0][w] >> k) & 1u);
        for (int p = 1; p < kMaxBits; ++p) {
          const int pos = sbp[p * D + dim];
          if (pos >= 0) idx |= row_bit(trec, lane, pos, cv.code_bytes) << p;
        }
        const float c = scen[dim * kMaxLevels + idx];
        const bool og = k < cv.o4;
        const float co = og ? c : 0.f, cr = c - co;
        const float sgn = (sg[w] >> k) & 1u ? 1.f : -1.f;
        const float go = og ? sgn : 0.f, gr = sgn - go;
        const float4 q = sqr[dim], t = sqs[dim];
        ao.x = fmaf(q.x, co, ao.x); ao.y = fmaf(q.y, co, ao.y); ao.z = fmaf(q.z, co, ao.z); ao.w = fmaf(q.w, co, ao.w);
        ar.x = fmaf(q.x, cr, ar.x); ar.y = fmaf(q.y, cr, ar.y); ar.z = fmaf(q.z, cr, ar.z); ar.w = fmaf(q.w, cr, ar.w);
        so.x = fmaf(t.x, go, so.x); so.y = fmaf(t.y, go, so.y); so.z = fmaf(t.z, go, so.z); so.w = fmaf(t.w, go, so.w);
        sr.x = fmaf(t.x, gr, sr.x); sr.y = fmaf(t.y, gr, sr.y); sr.z = fmaf(t.z, gr, sr.z); sr.w = fmaf(t.w, gr, sr.w);
      }
    }
    if (v >= n) return;
    const auto h16 = [&](int off) { return f16_to_f32(*reinterpret_cast<const uint16_t*>(trec + off + 2 * lane)); };
    const float nxr = h16(cv.off_nx), nxo = h16(cv.off_nxo);
    const bool prod = cv.mode == TQ_PROD;
    const float kr = prod ? h16(cv.off_nr) * kQjl / float(D - 4 * cv.o4) : 0.f;
    const float ko = prod ? h16(cv.off_nro) * kQjl / float(4 * cv.o4) : 0.f;
    const float out[4] = {nxo * (ao.x + ko * so.x) + nxr * (ar.x + kr * sr.x),
                          nxo * (ao.y + ko * so.y) + nxr * (ar.y + kr * sr.y),
                          nxo * (ao.z + ko * so.z) + nxr * (ar.z + kr * sr.z),
                          nxo * (ao.w + ko * so.w) + nxr * (ar.w + kr * sr.w)};
#pragma unroll
    for (int qq = 0; qq < QB; ++qq)
      if (qq < nqb) scores[(q0 + qq) * n + v] = out[qq];
    return;
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      const int dim = 32 * w + k;
      int idx = 0;
#pragma unroll
      for (int p = 0; p < kMaxBits; ++p)
        if (p < np) idx |= int((pl[p][w] >> k) & 1u) << p;
      float c;
      if (cv.uniform) {
        c = scen[idx];
      } else {
        for (int p = 1; p < kMaxBits; ++p) {
          const int pos = cv.bitpos[p * D + dim];
          if (pos >= 0) idx |= int((tail >> (pos - D)) & 1u) << p;
        }
        c = scen[dim * kMaxLevels + idx];
      }
      const float4 q = sqr[dim];
      acc.x = fmaf(q.x, c, acc.x);
      acc.y = fmaf(q.y, c, acc.y);
      acc.z = fmaf(q.z, c, acc.z);
      acc.w = fmaf(q.w, c, acc.w);
    }
  }
  float4 sacc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (cv.mode == TQ_PROD) {
    if (m == D) {
      const u32x4 sg = *reinterpret_cast<const u32x4*>(trec + cv.off_signs + size_t(lane) * 16);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll 8
        for (int k = 0; k < 32; ++k) {
          const float sgn = (sg[w] >> k) & 1u ? 1.f : -1.f;
          const float4 q = sqs[32 * w + k];
          sacc.x = fmaf(q.x, sgn, sacc.x);
          sacc.y = fmaf(q.y, sgn, sacc.y);
          sacc.z = fmaf(q.z, sgn, sacc.z);
          sacc.w = fmaf(q.w, sgn, sacc.w);
        }
      }
    } else {
      uint32_t sg = 0;
      for (int k = 0; k < cv.sign_bytes; ++k)
        sg |= uint32_t(trec[cv.off_signs + size_t(lane) * cv.sign_bytes + k]) << (8 * k);
      for (int jrow = 0; jrow < m; ++jrow) {
        const float sgn = (sg >> jrow) & 1u ? 1.f : -1.f;
        const float4 q = sqs[jrow];
        sacc.x = fmaf(q.x, sgn, sacc.x);
        sacc.y = fmaf(q.y, sgn, sacc.y);
        sacc.z = fmaf(q.z, sgn, sacc.z);
        sacc.w = fmaf(q.w, sgn, sacc.w);
      }
    }
  }
  if (v >= n) return;
  const float nx = f16_to_f32(*reinterpret_cast<const uint16_t*>(trec + cv.off_nx + 2 * lane));
  const float nr = cv.mode == TQ_PROD
                       ? f16_to_f32(*reinterpret_cast<const uint16_t*>(trec + cv.off_nr + 2 * lane))
                       : 0.f;
  const float coef = cv.mode == TQ_PROD ? nr * kQjl / float(m) : 0.f;
  const float out[4] = {acc.x + coef * sacc.x, acc.y + coef * sacc.y, acc.z + coef * sacc.z,
                        acc.w + coef * sacc.w};
#pragma unroll
  for (int qq = 0; qq < QB; ++qq)
    if (qq < nqb) scores[(q0 + qq) * n + v] = nx * out[qq];
}

// ------------------------------------------------------------ decode
// Split-K partial: block (split, kv head g, sequence b), 4 waves each taking
// tiles of the split in turn.  Partial record per (b, g, split):
// [G] max, [G] sum, [G][128] accumulator.
template <int G>
__global__ __launch_bounds__(256) void decode_partial_kernel(CodecView kc, CodecView vc, DecodeArgs a) {
  constexpr int D = 128;
  __shared__ float sqr[G][D];
  __shared__ float sqs[G][D];
  __shared__ float skcen[D * kMaxLevels];
  __shared__ float svcen[D * kMaxLevels];  // uniform values: the first kMaxLevels
  __shared__ float spw[4][G][kTile];
  __shared__ float spwo[4][G][kTile];  // split values: weights times the outlier group's norm
  __shared__ float sm_m[4][G], sm_l[4][G];
  __shared__ float sacc[4][G][D];
  __shared__ int16_t sbp[kMaxBits * D];  // split keys: bit positions of the index bits
  __shared__ int16_t svbp[kMaxBits * D];  // non-uniform ROW values: bit positions of the index bits

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int mk = kc.mode == TQ_PROD ? kc.m : 0;
  if (kc.outl)
    for (int e = threadIdx.x; e < kMaxBits * D; e += blockDim.x) sbp[e] = kc.bitpos[e];
  const int hk = kc.heads > 1 ? g : 0, hv = vc.heads > 1 ? g : 0;
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int gg = e / D, i = e % D;
    const int64_t qi = (int64_t(b) * a.Hq + g * G + gg);
    sqr[gg][i] = a.qr[qi * D + i];
    sqs[gg][i] = i < mk ? a.qs[qi * mk + i] : 0.f;
  }
  if (kc.uniform) {
    for (int e = threadIdx.x; e < kMaxLevels; e += blockDim.x) skcen[e] = kc.ucen[e];
  } else {
    for (int e = threadIdx.x; e < D * kMaxLevels; e += blockDim.x)
      skcen[e] = kc.cen[size_t(hk) * D * kMaxLevels + e];
  }
  if (vc.uniform) {
    for (int e = threadIdx.x; e < kMaxLevels; e += blockDim.x) svcen[e] = vc.ucen[e];
  } else {
    for (int e = threadIdx.x; e < D * kMaxLevels; e += blockDim.x)
      svcen[e] = vc.cen[size_t(hv) * D * kMaxLevels + e];
    for (int e = threadIdx.x; e < kMaxBits * D; e += blockDim.x) svbp[e] = vc.bitpos[e];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int len = a.seq_lens ? min(a.seq_lens[b] + a.len_add, a.max_tokens) : a.max_tokens;
  const int ntiles = (len + kTile - 1) / kTile;
  const uint8_t* kbase = a.krec + int64_t(b) * a.ks_seq + int64_t(g) * a.ks_head;
  const uint8_t* vbase = a.vrec + int64_t(b) * a.vs_seq + int64_t(g) * a.vs_head;

  float mrun[G], lrun[G], acc0[G], acc1[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) { mrun[gg] = -INFINITY; lrun[gg] = 0.f; acc0[gg] = acc1[gg] = 0.f; }

  const int t_begin = split * a.chunk_tiles;
  const int t_end = min(ntiles, t_begin + a.chunk_tiles);
  for (int tile = t_begin + wave; tile < t_end; tile += 4) {
    const uint8_t* kt = kbase + int64_t(tile) * kc.tile_bytes;
    const uint8_t* vt = vbase + int64_t(tile) * vc.tile_bytes;
    if (a.block_table) {
      const int64_t pt = paged_tile(a.block_table, a.page_shift, a.max_pages, int64_t(b) * a.Hkv + g, tile);
      kt = a.krec + pt * kc.tile_bytes;
      vt = a.vrec + pt * vc.tile_bytes;
    }
    const int tok = tile * kTile + lane;
    const bool valid = tok < len;
    // ---- scores (lane = token)
    float sc[G];  // estimated <q, k> per query
    if (kc.outl) {
      // outlier-channel split: stored coordinate i is an outlier one when
      // i % 32 < o4; each group has its own norms and QJL factor
      float so[G], sr[G], go[G], gr[G];
#pragma unroll
      for (int gg = 0; gg < G; ++gg) so[gg] = sr[gg] = go[gg] = gr[gg] = 0.f;
      for (int dim = 0; dim < D; ++dim) {
        int idx = (kt[size_t(lane) * 16 + (dim >> 3)] >> (dim & 7)) & 1;
        for (int p = 1; p < kMaxBits; ++p) {
          const int pos = sbp[p * D + dim];
          if (pos >= 0) idx |= row_bit(kt, lane, pos, kc.code_bytes) << p;
        }
        const float c = skcen[dim * kMaxLevels + idx];
        const bool og = (dim & 31) < kc.o4;
        float sgn = 0.f;
        if (kc.mode == TQ_PROD) sgn = (kt[kc.off_signs + size_t(lane) * 16 + (dim >> 3)] >> (dim & 7)) & 1 ? 1.f : -1.f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const float qc = sqr[gg][dim] * c, qg = sqs[gg][dim] * sgn;
          if (og) { so[gg] += qc; go[gg] += qg; } else { sr[gg] += qc; gr[gg] += qg; }
        }
      }
      const auto h16 = [&](int off) { return f16_to_f32(*reinterpret_cast<const uint16_t*>(kt + off + 2 * lane)); };
      const bool prod = kc.mode == TQ_PROD;
      const float nxr = h16(kc.off_nx), nxo = h16(kc.off_nxo);
      const float kr = prod ? h16(kc.off_nr) * kQjl / float(D - 4 * kc.o4) : 0.f;
      const float ko = prod ? h16(kc.off_nro) * kQjl / float(4 * kc.o4) : 0.f;
#pragma unroll
      for (int gg = 0; gg < G; ++gg) sc[gg] = nxo * (so[gg] + ko * go[gg]) + nxr * (sr[gg] + kr * gr[gg]);
    } else {
    float s[G], sg[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) s[gg] = sg[gg] = 0.f;
    for (int dim = 0; dim < D; ++dim) {
      int idx;
      float c;
      if (kc.uniform) {
        idx = row_index_uniform(kt, lane, dim, D, kc.ubits);
        c = skcen[idx];
      } else {
        idx = (kt[size_t(lane) * 16 + (dim >> 3)] >> (dim & 7)) & 1;
        for (int p = 1; p < kMaxBits; ++p) {
          const int pos = kc.bitpos[p * D + dim];
          if (pos >= 0) {
            const int tb = kc.code_bytes - 16, t = pos - D;
            idx |= ((kt[size_t(kTile) * 16 + size_t(lane) * tb + (t >> 3)] >> (t & 7)) & 1) << p;
          }
        }
        c = skcen[dim * kMaxLevels + idx];
      }
#pragma unroll
      for (int gg = 0; gg < G; ++gg) s[gg] = fmaf(sqr[gg][dim], c, s[gg]);
    }
    float coef = 0.f;
    if (kc.mode == TQ_PROD) {
      for (int jrow = 0; jrow < mk; ++jrow) {
        int bit;
        if (mk > 8)
          bit = (kt[kc.off_signs + size_t(lane) * 16 + (jrow >> 3)] >> (jrow & 7)) & 1;
        else
          bit = (kt[kc.off_signs + size_t(lane) * kc.sign_bytes] >> jrow) & 1;
        const float sgn = bit ? 1.f : -1.f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) sg[gg] = fmaf(sqs[gg][jrow], sgn, sg[gg]);
      }
      coef = f16_to_f32(*reinterpret_cast<const uint16_t*>(kt + kc.off_nr + 2 * lane)) * kQjl / float(mk);
    }
    const float nx = f16_to_f32(*reinterpret_cast<const uint16_t*>(kt + kc.off_nx + 2 * lane));
#pragma unroll
    for (int gg = 0; gg < G; ++gg) sc[gg] = nx * (s[gg] + coef * sg[gg]);
    }
    const float nv = f16_to_f32(*reinterpret_cast<const uint16_t*>(vt + vc.off_nx + 2 * lane));
    const float nvo = vc.outl ? f16_to_f32(*reinterpret_cast<const uint16_t*>(vt + vc.off_nxo + 2 * lane)) : 0.f;
    // ---- online softmax
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float logit = valid ? a.scale * sc[gg] : -INFINITY;
      const float mt = wave_max(logit);
      const float mnew = fmaxf(mrun[gg], mt);
      const float alpha = mrun[gg] == -INFINITY ? 0.f : __expf(mrun[gg] - mnew);
      const float p = valid ? __expf(logit - mnew) : 0.f;
      lrun[gg] = lrun[gg] * alpha + wave_sum(p);
      acc0[gg] *= alpha;
      acc1[gg] *= alpha;
      mrun[gg] = mnew;
      spw[wave][gg][lane] = p * nv;
      if (vc.outl) spwo[wave][gg][lane] = p * nvo;
    }
    __builtin_amdgcn_wave_barrier();
    // ---- values (lane = dims lane, lane + 64)
    if (vc.layout == TQ_LAYOUT_ROW) {
      // row records (any uniform codec, or a split one): the index of
      // (token t, stored coordinate i) from the planes of t's row; a split
      // codec scales each coordinate by its group's norm (stored coordinate
      // i is an outlier one when i % 32 < o4, the same for i and i + 64)
      const bool og = vc.outl && (lane & 31) < vc.o4;
      const float(*w_)[kTile] = og ? spwo[wave] : spw[wave];
      auto vidx = [&](int t, int dim) -> int {
        if (vc.uniform) return row_index_uniform(vt, t, dim, D, vc.ubits);
        int idx = (vt[size_t(t) * 16 + (dim >> 3)] >> (dim & 7)) & 1;
        for (int p = 1; p < kMaxBits; ++p) {
          const int pos = svbp[p * D + dim];
          if (pos >= 0) idx |= row_bit(vt, t, pos, vc.code_bytes) << p;
        }
        return idx;
      };
      const int l0 = vc.uniform ? 0 : lane * kMaxLevels, l1 = vc.uniform ? 0 : (lane + 64) * kMaxLevels;
      for (int t = 0; t < kTile; ++t) {
        const float c0 = svcen[l0 + vidx(t, lane)], c1 = svcen[l1 + vidx(t, lane + 64)];
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const float w = w_[gg][t];
          acc0[gg] = fmaf(w, c0, acc0[gg]);
          acc1[gg] = fmaf(w, c1, acc1[gg]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      continue;
    }
    // index-major col fields
    const int vb = vc.ubits;
    const uint8_t* f0 = vt + size_t(lane) * 8 * vb;
    const uint8_t* f1 = vt + size_t(lane + 64) * 8 * vb;
    for (int t = 0; t < kTile; ++t) {
      const int bit = vb * t;
      const int i0 = int(((uint32_t(f0[bit >> 3]) | (uint32_t(f0[min((bit >> 3) + 1, 8 * vb - 1)]) << 8)) >> (bit & 7)) & ((1u << vb) - 1));
      const int i1 = int(((uint32_t(f1[bit >> 3]) | (uint32_t(f1[min((bit >> 3) + 1, 8 * vb - 1)]) << 8)) >> (bit & 7)) & ((1u << vb) - 1));
      const float c0 = svcen[i0], c1 = svcen[i1];
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const float w = spw[wave][gg][t];
        acc0[gg] = fmaf(w, c0, acc0[gg]);
        acc1[gg] = fmaf(w, c1, acc1[gg]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // ---- merge the 4 waves
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    if (lane == 0) { sm_m[wave][gg] = mrun[gg]; sm_l[wave][gg] = lrun[gg]; }
    sacc[wave][gg][lane] = acc0[gg];
    sacc[wave][gg][lane + 64] = acc1[gg];
  }
  __syncthreads();
  float* out = a.part + ((int64_t(b) * a.Hkv + g) * a.nsplit + split) * (G * (2 + D));
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int gg = e / D, i = e % D;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][gg]);
    float accv = 0.f, l = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = sm_m[w][gg] == -INFINITY ? 0.f : __expf(sm_m[w][gg] - M);
      accv += f * sacc[w][gg][i];
      l += f * sm_l[w][gg];
    }
    out[2 * G + gg * D + i] = accv;
    if (i == 0) { out[gg] = M; out[G + gg] = l; }
  }
}

// Merge of the splits and inverse value rotation: block (query head, b).
// Up to 64 splits (the usual case) every load -- the split maxima and sums,
// the partial accumulators and the rotation columns -- is issued at once, so
// the kernel costs one memory round trip plus LDS reductions; more splits
// take a loop over them.
template <int G>
__global__ __launch_bounds__(256) void decode_combine_kernel(CodecView vc, DecodeArgs a) {
  // One block per (sequence, query head): merge the split-K partials
  // (log-sum-exp), then rotate back, out = Pi_v^T acc / l.  Thread t takes
  // coordinate i = t % 128 over half h = t / 128 of the splits and of the
  // rotation's k range.
  constexpr int D = 128;
  constexpr int kFast = 64;
  __shared__ float sy[2][D];
  __shared__ float sf[1024];
  __shared__ float sred[8];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int g = hq / G, gg = hq % G;
  const int stride = G * (2 + D);
  const float* part = a.part + (int64_t(b) * a.Hkv + g) * a.nsplit * stride;
  const int t = threadIdx.x, i = t & (D - 1), half = t >> 7, lane = t & 63, wv = t >> 6;
  const int ns = min(a.nsplit, 1024);
  // rotation columns: out_i = sum_k Pi[k][i] y_k, k in this half
  const int hv = vc.heads > 1 ? g : 0;
  const float* rot = vc.rot + size_t(hv) * D * D + size_t(64 * half) * D + i;
  const bool had = vc.had_sign != nullptr;  // randomized Hadamard: out = s (H y) / sqrt(d)
  float r[64];
  if (!had) {
#pragma unroll
    for (int u = 0; u < 64; ++u) r[u] = rot[size_t(u) * D];
  }
  const float* pa = part + 2 * G + gg * D + i;
  float accv = 0.f, M, l;
  if (ns <= kFast) {
    // wave 0: split maxima; wave 1: split sums; every thread: its half's
    // accumulator entries (splits half, half + 2, ...)
    const float mv = (wv == 0 && lane < ns) ? part[lane * stride + gg] : -INFINITY;
    const float lv = (wv == 1 && lane < ns) ? part[lane * stride + G + gg] : 0.f;
    float v[kFast / 2];
#pragma unroll
    for (int u = 0; u < kFast / 2; ++u) v[u] = half + 2 * u < ns ? pa[(half + 2 * u) * stride] : 0.f;
    float m = mv;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (t == 0) sred[0] = m;
    __syncthreads();
    M = sred[0];
    // weights exp(m_s - M) of the splits (a split without tokens has m = -inf)
    if (wv == 0) {
      const float f = mv == -INFINITY ? 0.f : __expf(mv - M);
      sf[lane] = f;
    }
    __syncthreads();
    if (wv == 1) {
      float lp = sf[lane] * lv;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) lp += __shfl_xor(lp, o, 64);
      if (lane == 0) sred[1] = lp;
    }
#pragma unroll
    for (int u = 0; u < kFast / 2; ++u) accv = fmaf(sf[(half + 2 * u) & (kFast - 1)], v[u], accv);
    __syncthreads();
    l = sred[1];
  } else {
    float mx = -INFINITY;
    for (int s2 = t; s2 < ns; s2 += 256) {
      const float m = part[s2 * stride + gg];
      sf[s2] = m;
      mx = fmaxf(mx, m);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) sred[wv] = mx;
    __syncthreads();
    M = fmaxf(fmaxf(sred[0], sred[1]), fmaxf(sred[2], sred[3]));
    float lpart = 0.f;
    for (int s2 = t; s2 < ns; s2 += 256) {
      const float f = sf[s2] == -INFINITY ? 0.f : __expf(sf[s2] - M);
      sf[s2] = f;
      lpart += f * part[s2 * stride + G + gg];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lpart += __shfl_xor(lpart, o, 64);
    __syncthreads();
    if (lane == 0) sred[4 + wv] = lpart;
    __syncthreads();
    l = sred[4] + sred[5] + sred[6] + sred[7];
    int s2 = half;
    for (; s2 + 30 < ns; s2 += 32) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = pa[(s2 + 2 * u) * stride];
#pragma unroll
      for (int u = 0; u < 16; ++u) accv = fmaf(sf[s2 + 2 * u], v[u], accv);
    }
    for (; s2 < ns; s2 += 2) accv = fmaf(sf[s2], pa[s2 * stride], accv);
  }
  sy[half][i] = accv;
  __syncthreads();
  if (half == 0) sy[0][i] = l > 0.f ? (sy[0][i] + sy[1][i]) / l : 0.f;
  __syncthreads();
  if (had) {
    if (wv == 0) {
      float lo = sy[0][lane], hi = sy[0][lane + 64];
      fwht128_wave(lo, hi, lane);
      float* o = a.out + (int64_t(b) * a.Hq + hq) * D;
      o[lane] = vc.had_sign[lane] * lo * kInvSqrt128;
      o[lane + 64] = vc.had_sign[lane + 64] * hi * kInvSqrt128;
    }
    return;
  }
  const float* yk = sy[0] + 64 * half;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 64; ++u) o[u & 3] = fmaf(r[u], yk[u], o[u & 3]);
  __syncthreads();
  if (half == 1) sy[1][i] = (o[0] + o[1]) + (o[2] + o[3]);
  __syncthreads();
  if (half == 0) a.out[(int64_t(b) * a.Hq + hq) * D + i] = (o[0] + o[1]) + (o[2] + o[3]) + sy[1][i];
}

// ------------------------------------------------------------------ top-k
__device__ __forceinline__ bool better(float s1, int64_t i1, float s2, int64_t i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

// One wave per (query, segment).  The wave keeps one sorted top-16 list
// spread over the 16 lanes of each row (lane i of every row holds entry i;
// the four rows stay identical).  The segment is scanned 256 scores at a
// time; a score enters only if it beats the list's k-th entry (the running
// threshold), and entering candidates are inserted one at a time with a row
// shift, so after the first few blocks almost every block is a compare and a
// ballot.  Scores are part[q][t] * row_scale[q] * col_scale[t] (scales
// optional).  Lanes 0..k-1 write the segment's sorted top-k.
__global__ __launch_bounds__(256) void topk_segment_kernel(const float* scores, int64_t ld,
                                                           int64_t cols, int64_t id_base, int k,
                                                           int nseg, int seg_base, int total_seg,
                                                           float* ps, int64_t* pi,
                                                           const float* col_scale,
                                                           const float* row_scale) {
  const int lane = threadIdx.x & 63, li16 = lane & 15;
  const int seg = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t qi = blockIdx.y;
  if (seg >= nseg) return;
  const int64_t per = (cols + nseg - 1) / nseg;
  const int64_t lo = seg * per, hi = min(cols, lo + per);
  const float* row = scores + qi * ld;
  const float rsc = row_scale ? row_scale[qi] : 1.f;
  float Ls = -INFINITY;        // entry li16 of the list
  int64_t Lid = INT64_MAX;
  float ts = -INFINITY;        // threshold: entry k-1
  int64_t tid = INT64_MAX;
  for (int64_t base = lo; base < hi; base += 256) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = base + 64 * u + lane;
      v[u] = t < hi ? row[t] * rsc * (col_scale ? col_scale[t] : 1.f) : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = base + 64 * u + lane;
      const int64_t id = id_base + t;
      bool pend = t < hi;
      while (true) {
        const uint64_t m = __ballot(pend && better(v[u], id, ts, tid));
        if (m == 0) break;
        const int src = __ffsll((unsigned long long)m) - 1;
        const float cs = __shfl(v[u], src, 64);
        const int64_t cid = id_base + base + 64 * u + src;
        // insert (cs, cid): entries better than it keep their place
        const bool keep = better(Ls, Lid, cs, cid);
        const int pos = __popcll(__ballot(keep) & 0xffffull);
        const float shs = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(Ls), __float_as_int(Ls),
                                                                     0x111, 0xF, 0xF, false));  // row_shr:1
        const uint32_t idl = uint32_t(uint64_t(Lid)), idh = uint32_t(uint64_t(Lid) >> 32);
        const uint32_t shl = uint32_t(__builtin_amdgcn_update_dpp(int(idl), int(idl), 0x111, 0xF, 0xF, false));
        const uint32_t shh = uint32_t(__builtin_amdgcn_update_dpp(int(idh), int(idh), 0x111, 0xF, 0xF, false));
        if (!keep) {
          if (li16 == pos) { Ls = cs; Lid = cid; }
          else { Ls = shs; Lid = int64_t((uint64_t(shh) << 32) | shl); }
        }
        ts = __shfl(Ls, k - 1, 64);
        tid = __shfl(Lid, k - 1, 64);
        if (lane == src) pend = false;
      }
    }
  }
  if (lane < k) {
    const int64_t o = (qi * total_seg + seg_base + seg) * k + lane;
    ps[o] = Ls;
    pi[o] = Lid;
  }
}

// One wave per query: k rounds of a wave-wide argmax over the heads of the
// sorted partial lists (lane j owns lists j, j + 64, ...).
__global__ __launch_bounds__(64) void topk_merge_kernel(const float* ps, const int64_t* pi,
                                                        int nseg, int k, float* out_s,
                                                        int64_t* out_i) {
  __shared__ int heads[1024];
  const int64_t qi = blockIdx.x;
  const int lane = threadIdx.x;
  for (int sg = lane; sg < nseg; sg += 64) heads[sg] = 0;
  __syncthreads();
  const float* qps = ps + qi * nseg * k;
  const int64_t* qpi = pi + qi * nseg * k;
  for (int r = 0; r < k; ++r) {
    float bs = -INFINITY;
    int64_t bi = INT64_MAX;
    int bseg = -1;
    for (int sg = lane; sg < nseg; sg += 64) {
      const int h = heads[sg];
      if (h >= k) continue;
      const float v = qps[sg * k + h];
      const int64_t id = qpi[sg * k + h];
      if (bseg < 0 || better(v, id, bs, bi)) { bs = v; bi = id; bseg = sg; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float os = __shfl_xor(bs, o, 64);
      const int64_t oi = __shfl_xor(bi, o, 64);
      const int oseg = __shfl_xor(bseg, o, 64);
      if (oseg >= 0 && (bseg < 0 || better(os, oi, bs, bi))) { bs = os; bi = oi; bseg = oseg; }
    }
    if (lane == 0) {
      out_s[qi * k + r] = bs;
      out_i[qi * k + r] = bi;
      if (bseg >= 0) ++heads[bseg];
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_query_prep(const CodecView& cv, const QueryPrepArgs& a, hipStream_t s) {
  // enough blocks to spread over the chip, up to 8 queries per Pi read
  int qb = 1;  // a power of two, so that a block never straddles two heads' query groups
  while (qb < 8 && int64_t(qb) * 2 * 512 <= a.nq) qb *= 2;
  if (a.q_per_head > 0) qb = std::min(qb, a.q_per_head & -a.q_per_head);
  if (cv.d != 128) return hipErrorNotSupported;
  const size_t lds = size_t(4) * qb * cv.d * 4;
  const unsigned blocks = unsigned((a.nq + qb - 1) / qb);
  hipLaunchKernelGGL(query_prep_kernel, dim3(blocks), dim3(256), lds, s, cv, a, qb);
  return hipGetLastError();
}

hipError_t launch_score(const CodecView& cv, const float* qr, const float* qs, int64_t nq,
                        const uint8_t* rec, int64_t n, float* scores, hipStream_t s, int head) {
  constexpr int QB = 4;
  if (cv.d != 128 || cv.layout != TQ_LAYOUT_ROW || (cv.uniform && cv.ubits > kMaxBits)) return hipErrorNotSupported;
  if (cv.outl && cv.mode == TQ_PROD && cv.m != 128) return hipErrorNotSupported;
  const int64_t ntiles = (n + kTile - 1) / kTile;
  dim3 grid(unsigned((ntiles + 3) / 4), unsigned((nq + QB - 1) / QB));
  hipLaunchKernelGGL(score_kernel<QB>, grid, dim3(256), 0, s, cv, qr, qs, nq, rec, n, scores, head);
  return hipGetLastError();
}

hipError_t launch_decode(const CodecView& kv, const CodecView& vv, const DecodeArgs& a,
                         hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  dim3 grid(unsigned(a.nsplit), unsigned(a.Hkv), unsigned(a.B));
  hipError_t e;
  if (decode_mfma_supported(kv, vv, G)) {
    e = launch_decode_mfma(kv, vv, a, s);
    // a single split is normalised and rotated back inside the MFMA kernel
    if (e != hipSuccess || a.nsplit == 1) return e;
  } else {
    switch (G) {
      case 1: hipLaunchKernelGGL(decode_partial_kernel<1>, grid, dim3(256), 0, s, kv, vv, a); break;
      case 2: hipLaunchKernelGGL(decode_partial_kernel<2>, grid, dim3(256), 0, s, kv, vv, a); break;
      case 4: hipLaunchKernelGGL(decode_partial_kernel<4>, grid, dim3(256), 0, s, kv, vv, a); break;
      case 8: hipLaunchKernelGGL(decode_partial_kernel<8>, grid, dim3(256), 0, s, kv, vv, a); break;
      default: return hipErrorNotSupported;
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  dim3 g2(unsigned(a.Hq), unsigned(a.B));
  switch (G) {
    case 1: hipLaunchKernelGGL(decode_combine_kernel<1>, g2, dim3(256), 0, s, vv, a); break;
    case 2: hipLaunchKernelGGL(decode_combine_kernel<2>, g2, dim3(256), 0, s, vv, a); break;
    case 4: hipLaunchKernelGGL(decode_combine_kernel<4>, g2, dim3(256), 0, s, vv, a); break;
    case 8: hipLaunchKernelGGL(decode_combine_kernel<8>, g2, dim3(256), 0, s, vv, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_topk_segments(const float* scores, int64_t ld, int64_t cols, int64_t id_base,
                                int64_t nq, int k, int nseg, int seg_base, int total_seg,
                                float* ps, int64_t* pi, hipStream_t s, const float* col_scale,
                                const float* row_scale) {
  hipLaunchKernelGGL(topk_segment_kernel, dim3(unsigned((nseg + 3) / 4), unsigned(nq)), dim3(256), 0, s,
                     scores, ld, cols, id_base, k, nseg, seg_base, total_seg, ps, pi, col_scale, row_scale);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const float* ps, const int64_t* pi, int64_t nq, int total_seg, int k,
                             float* out_s, int64_t* out_i, hipStream_t s) {
  hipLaunchKernelGGL(topk_merge_kernel, dim3(unsigned(nq)), dim3(64), 0, s, ps, pi, total_seg, k, out_s,
                     out_i);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace tq
