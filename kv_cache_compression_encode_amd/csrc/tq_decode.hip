// Fused decode attention over a compressed KV cache on MFMA (gfx950), d = 128.
//
// Keys: TurboQuant-prod row records with 1 or 2 index bits.  A symmetric
// Lloyd-Max codebook with 4 levels is exactly linear in the two bit planes
// written as signs s = 2b - 1:  c(idx) = alpha s1 + beta s0 with
// alpha = (c3 + c2)/2, beta = (c3 - c2)/2 (2 levels: c(idx) = c1 s0).  So the
// score of a query against a key,
//   n_x ( <q', c(idx)> + n_r sqrt(pi/2)/m <qs, sign> ),
// is one contraction over K = [plane 0 | plane 1 | signs] (3 x 128) of +-1
// values with the weighted query: a single chain of 16x16x32 f16 MFMAs per 16
// keys.  Rows 0..7 carry the code part of 4 queries (fp16 hi and lo parts of
// w_p q'), rows 8..15 the sign part (hi and lo of qs); each +-1 operand (8
// fp16 values for 8 key bits) is one 16-byte read of a 256-entry LDS table
// indexed by the key byte.
//
// SpectralQuant keys (UB = 0): dims 4..127 carry one bit each, so their part
// of <q', c(idx)> is linear in plane 0 (c_i(b) = mu_i + gamma_i s) and runs
// on the same MFMA chain (rows 0..7 only); the multi-bit dims 0..3 (index bits
// in plane 0 plus the tail byte) read a per-query LDS table of q'_i c_i(idx),
// and the 4 QJL signs are a 4-term dot product on the VALU.
//
// Outlier-channel split keys (UB = 3): stored coordinates 32 g + s, s < 8,
// are the outlier instance's (2 index bits, levels alpha s1 + beta s0); the
// rest are regular (1 bit, c_1 s0).  In every MFMA of the chain chunk c = 0
// holds exactly the outlier coordinates, so the outlier and regular parts
// accumulate in two chains: plane 0 (4 chunks), plane 1 (its 32 bits: chunk 0
// only) and the signs (4 chunks), 9 MFMAs per 16 keys; each part is then
// scaled by its own group's norms and QJL factor.
//
// Values: TurboQuant-mse col records with 4 index bits: 8 consecutive tokens
// of one coordinate are one dword; a 256-entry LDS table maps each byte (two
// tokens) to the fp16 pair of their centroids, giving the B operand of
// P V_hat directly (P = softmax weights times n_v, fp16, rows = queries).
//
// Online softmax per query over 64-token tiles; split-K over tiles with the
// same partial format as the generic kernel, merged by decode_combine.
#include <hip/hip_runtime.h>

#include <cmath>

#include "tq_kernels.h"

namespace tq {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr float kQjl = 1.2533141373155001f;  // sqrt(pi / 2)

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t f16b(float x) {
  return uint32_t(__builtin_bit_cast(uint16_t, (_Float16)x));
}
__device__ __forceinline__ float f16v(uint32_t h) {
  return float(__builtin_bit_cast(_Float16, uint16_t(h)));
}
__device__ __forceinline__ float h2f(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }

// Reductions over the 16 lanes of a row with DPP row rotations (no LDS
// round trips), and exchanges with the lane 32 (or 16) positions away with
// the gfx950 permlane swaps.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ __forceinline__ float grp_max(float v) {
  v = fmaxf(v, dpp<0x128>(v));  // row_ror:8
  v = fmaxf(v, dpp<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp<0x122>(v));  // row_ror:2
  return fmaxf(v, dpp<0x121>(v));  // row_ror:1
}
__device__ __forceinline__ float grp_sum(float v) {
  v += dpp<0x128>(v);
  v += dpp<0x124>(v);
  v += dpp<0x122>(v);
  return v + dpp<0x121>(v);
}
__device__ __forceinline__ float xor32(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}
// 4 x 4 transpose of (16-lane row, register): on return register k of row r
// holds register r of row k (two permlane16 swaps, then two permlane32 swaps).
__device__ __forceinline__ u32x4 transpose4(u32x4 m, int lane) {
  (void)lane;
  auto a = __builtin_amdgcn_permlane16_swap(m[0], m[1], false, false);
  auto b = __builtin_amdgcn_permlane16_swap(m[2], m[3], false, false);
  auto c = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
  return u32x4{c[0], d[0], c[1], d[1]};
}

__device__ __forceinline__ float xor16(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane & 16) ? r[0] : r[1]);
}

template <int G, int UB>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(CodecView kc, CodecView vc, DecodeArgs a) {
  static_assert(G >= 1 && G <= 4, "up to 4 query heads per KV head");
  constexpr bool SQ = UB == 0;
  constexpr bool SPL = UB == 3;  // outlier-channel split keys, 32 outlier coordinates
  __shared__ float sqr[4][D];
  __shared__ float sqs[4][D];
  __shared__ float slow[SQ ? 4 : 1][4][kMaxLevels];  // SQ: q'_i c_i(idx), dims 0..3
  __shared__ float smu[4];
  __shared__ float sgam[SQ ? D : 1], smuv[SQ ? D : 1];  // SQ: one-bit dims' (c1 - c0)/2, (c1 + c0)/2
  __shared__ uint32_t stail[SQ ? 256 : 1];  // SQ: tail byte -> index bits 1.. of dims 0..3 (5 bits each)
  __shared__ float skc[SQ ? 4 : 1][kMaxLevels];  // SQ: levels of dims 0..3
  // value byte (two 4-bit codes) -> fp16 pair of their levels, 32 copies:
  // entry e for lane l at slut[e * 32 + l % 32], so that the random lookups
  // of a wave hit 32 distinct banks
  __shared__ uint32_t slut1[256];
  __shared__ uint32_t slut[256 * 32];
  constexpr int PROW = 64 + 8;  // padded row of the P buffer (bank spread)
  __shared__ __align__(16) uint16_t sP[4][16][PROW];  // per wave: [query row][token] fp16 weights
  __shared__ float sm_m[4][4], sm_l[4][4];
  __shared__ float sacc[4][4][D];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g16 = lane >> 4;
  const int len = a.seq_lens ? min(a.seq_lens[b] + a.len_add, a.max_tokens) : a.max_tokens;
  const int ntiles = (len + kTile - 1) / kTile;
  const uint8_t* kbase = a.krec + int64_t(b) * a.ks_seq + int64_t(g) * a.ks_head;
  const uint8_t* vbase = a.vrec + int64_t(b) * a.vs_seq + int64_t(g) * a.vs_head;
  const int t_begin = split * a.chunk_tiles;
  const int t_end = min(ntiles, t_begin + a.chunk_tiles);
  constexpr int NP = SQ ? 1 : (SPL ? 3 : UB + 1);  // +-1 planes in the MFMA chain (incl. signs)
  // ---- loads of one tile: key planes/signs (dword g16 of token 16nb+n),
  // value fields, fp16 norms (raw), SQ low/tail/sign bytes; the next tile's
  // loads are issued before the current tile is processed
  // (raw values only: no ALU on loaded registers here, so the loads of the
  // next tile stay in flight while the current one is processed)
  // per-token words (norms, SQ bytes) are loaded once per token, by lane
  // (n, g16) for token 16 g16 + n, and shuffled to the lanes that use them
  // 16-byte loads: lane (n, g16) loads the whole 16-byte row of token
  // 16 g16 + n of each key plane, and 16 bytes of the value fields; a 4 x 4
  // transpose across the four 16-lane rows (permlane swaps) then gives every
  // lane the dwords its MFMA operands need.  One 16-byte load per lane moves
  // four times the data of a dword load through the address unit.
  struct TileRegs {
    u32x4 kw4[NP], vw4[4];
    uint32_t nx, nr, nv, tl, sg, xo, ro;
  };
  TileRegs cur, nxt;
  auto load_tile = [&](int tile, TileRegs& R) {
    const uint8_t* kt = kbase + int64_t(tile) * kc.tile_bytes;
    const uint8_t* vt = vbase + int64_t(tile) * vc.tile_bytes;
    if (a.block_table) {
      // the tile index is the wave's: one scalar read of the block table
      const int64_t pt = paged_tile(a.block_table, a.page_shift, a.max_pages, int64_t(b) * a.Hkv + g,
                                    __builtin_amdgcn_readfirstlane(tile));
      kt = a.krec + pt * kc.tile_bytes;
      vt = a.vrec + pt * vc.tile_bytes;
    }
    const int tok = 16 * g16 + n;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (SPL && p == 1) {
        // plane 1 of the split keys: one dword per token ([64][4] after plane 0)
        R.kw4[1][0] = *reinterpret_cast<const uint32_t*>(kt + kTile * 16 + tok * 4);
        continue;
      }
      const int off = SQ ? 0 : (p < (SPL ? 2 : UB) ? p * kTile * 16 : kc.off_signs);  // SQ: plane 0 only
      R.kw4[p] = *reinterpret_cast<const u32x4*>(kt + off + tok * 16);
    }
    // load j: dim 16 (2j + g16/2) + n, bytes 16 (g16 % 2) .. + 15 of its field
#pragma unroll
    for (int j = 0; j < 4; ++j)
      R.vw4[j] = *reinterpret_cast<const u32x4*>(vt + (16 * (2 * j + (g16 >> 1)) + n) * 32 + 16 * (g16 & 1));
    R.nx = *reinterpret_cast<const uint16_t*>(kt + kc.off_nx + 2 * tok);
    R.nr = *reinterpret_cast<const uint16_t*>(kt + kc.off_nr + 2 * tok);
    R.nv = *reinterpret_cast<const uint16_t*>(vt + vc.off_nx + 2 * tok);
    if (SQ) {
      R.tl = kt[kTile * 16 + tok];
      R.sg = kt[kc.off_signs + tok];
    }
    if (SPL) {
      R.xo = *reinterpret_cast<const uint16_t*>(kt + kc.off_nxo + 2 * tok);
      R.ro = *reinterpret_cast<const uint16_t*>(kt + kc.off_nro + 2 * tok);
    }
  };
  TileRegs& ra = cur;
  TileRegs& rb = nxt;
  // the first tile's loads go out before the set-up below and overlap it.
  // Contiguous records: they do not wait for seq_lens, since any tile below
  // max_tokens is in the records (a wave without a tile leaves them unused).
  // Paged records: only tiles below seq_lens are looked up in the block table
  // (the entries past them need not name pages).
  if (!a.block_table) {
    const int tmax = (a.max_tokens + kTile - 1) / kTile;
    load_tile(min(t_begin + wave, tmax - 1), ra);
  } else if (t_begin + wave < t_end) {
    load_tile(t_begin + wave, ra);
  }

  // ---- set-up: one round of independent loads, then arithmetic on LDS.
  // The G queries are rotated here, q' = Pi_h q and qs = S q'[0:m]: thread t
  // forms coordinate t % 128 over half t / 128 of each sum, reading the
  // transposed matrices column-coalesced (all their loads go out first).
  const int hk = kc.heads > 1 ? g : 0;
  const int ci = threadIdx.x & (D - 1), kh = threadIdx.x >> 7;
  float rcol[D / 2], scol[SQ ? 1 : D / 2];
  {
    const float* rt = kc.rot_t + size_t(hk) * D * D + size_t(kh * (D / 2)) * D + ci;
#pragma unroll
    for (int u = 0; u < D / 2; ++u) rcol[u] = rt[size_t(u) * D];
    if (!SQ) {
      const float* st = kc.sketch_t + size_t(kh * (D / 2)) * D + ci;
#pragma unroll
      for (int u = 0; u < D / 2; ++u) scol[u] = st[size_t(u) * D];
    }
  }
  for (int e = threadIdx.x; e < 4 * D; e += blockDim.x) {  // raw queries, staged in sqs
    const int gg = e / D, i = e % D;
    const int64_t qi = int64_t(b) * a.Hq + g * G + gg;
    float v = 0.f;
    if (gg < G)
      v = a.q_bf16 ? __uint_as_float(uint32_t(static_cast<const uint16_t*>(a.q)[qi * D + i]) << 16)
                   : static_cast<const float*>(a.q)[qi * D + i];
    sqs[gg][i] = v;
  }
  const float* kcen = kc.cen + size_t(hk) * D * kMaxLevels;
  {
    const int t = threadIdx.x;  // 256 threads: one value-table entry each
    slut1[t] = f16b(vc.ucen[t & 15]) | (f16b(vc.ucen[t >> 4]) << 16);
  }
  for (int e = threadIdx.x; e < 4 * 16 * PROW; e += blockDim.x) (&sP[0][0][0])[e] = 0;
  if (SQ) {
    stail[threadIdx.x] = kc.sq_tail[threadIdx.x];
    if (threadIdx.x < D) {
      sgam[threadIdx.x] = kc.sq_gm[(size_t(hk) * 2 + 0) * D + threadIdx.x];
      smuv[threadIdx.x] = kc.sq_gm[(size_t(hk) * 2 + 1) * D + threadIdx.x];
    } else {
      const int e = threadIdx.x - D;  // 128 threads: levels of dims 0..3
      skc[e / kMaxLevels][e % kMaxLevels] = kcen[(e / kMaxLevels) * kMaxLevels + e % kMaxLevels];
    }
  }
  __syncthreads();
  {
    // q' = Pi q: half sums into the (still unused) merge buffer, then added
    float* part = &sacc[0][0][0];  // [2][4][D]
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int u = 0; u < D / 2; u += 2) {
        s0 = fmaf(rcol[u], sqs[gg][kh * (D / 2) + u], s0);
        s1 = fmaf(rcol[u + 1], sqs[gg][kh * (D / 2) + u + 1], s1);
      }
      part[(kh * 4 + gg) * D + ci] = s0 + s1;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 4 * D; e += blockDim.x) sqr[e / D][e % D] = part[e] + part[4 * D + e];
    __syncthreads();
    if (!SQ) {
      // qs = S q' (m = d)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int u = 0; u < D / 2; u += 2) {
          s0 = fmaf(scol[u], sqr[gg][kh * (D / 2) + u], s0);
          s1 = fmaf(scol[u + 1], sqr[gg][kh * (D / 2) + u + 1], s1);
        }
        part[(kh * 4 + gg) * D + ci] = s0 + s1;
      }
      __syncthreads();
      for (int e = threadIdx.x; e < 4 * D; e += blockDim.x) sqs[e / D][e % D] = part[e] + part[4 * D + e];
    } else {
      // qs = S q'[0:m], m <= 4 (entries past m are zero)
      for (int e = threadIdx.x; e < 4 * D; e += blockDim.x) {
        const int gg = e / D, j = e % D;
        float acc = 0.f;
        if (j < kc.m)
          for (int k = 0; k < kc.m; ++k) acc = fmaf(kc.sketch[j * kc.m + k], sqr[gg][k], acc);
        sqs[gg][j] = acc;
      }
    }
    __syncthreads();
  }
#pragma unroll 8
  for (int k = 0; k < 32; ++k) {  // consecutive threads write consecutive words
    const int e = k * 256 + threadIdx.x;
    slut[e] = slut1[e >> 5];
  }
  if (SQ) {
    for (int e = threadIdx.x; e < 4 * 4 * kMaxLevels; e += blockDim.x) {
      const int gg = e / (4 * kMaxLevels), i = (e / kMaxLevels) % 4, l = e % kMaxLevels;
      slow[gg][i][l] = sqr[gg][i] * skc[i][l];
    }
    {  // wave w: sum_{i >= 4} mu_i q'_i of query w
      float v = 0.f;
      for (int i = 4 + lane; i < D; i += 64) v += smuv[i] * sqr[wave][i];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      if (lane == 0) smu[wave] = v;
    }
  }

  // ---- score A fragments: chunk (p, c): lane row r = n, dims 32 g16 + 8c + s
  float wp[2];
  // split keys: outlier alpha, beta (dim 0's 4 levels), regular c_1 (dim 8)
  float spl_a = 0.f, spl_b = 0.f, spl_c1 = 0.f;
  if (SPL) {
    const float* ce = kc.cen + size_t(hk) * D * kMaxLevels;
    spl_a = 0.5f * (ce[3] + ce[2]);
    spl_b = 0.5f * (ce[3] - ce[2]);
    spl_c1 = ce[8 * kMaxLevels + 1];
  }
  if (SQ || SPL) {
    wp[0] = wp[1] = 0.f;
  } else if (UB == 2) {
    wp[0] = 0.5f * (kc.ucen[3] - kc.ucen[2]);
    wp[1] = 0.5f * (kc.ucen[3] + kc.ucen[2]);
  } else {
    wp[0] = kc.ucen[1];
    wp[1] = 0.f;
  }
  // the A fragments depend on the lane only: the waves build them once into
  // LDS (fragment f by wave f % 4) and read them back per tile (keeping them
  // live across the tile loop would exceed the register budget)
  __shared__ u32x4 sA[NP * 4][64];
  // byte -> 8 fp16 +-1 values (element k from bit k): the B operands of the
  // score chain are read from this table instead of being expanded on the VALU
  __shared__ u32x4 spm[256];
  {
    const uint32_t e = threadIdx.x;
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = (((e >> (2 * j)) & 1u) ? 0x3C00u : 0xBC00u) | ((((e >> (2 * j + 1)) & 1u) ? 0x3C00u : 0xBC00u) << 16);
    spm[e] = r;
  }
  for (int f = wave; f < NP * 4; f += 4) {
    const int p = f / 4, c = f % 4;
    const bool sign_part = p == NP - 1;
    const int r = n;
    const bool rowsig = r >= 8;
    const int gq = (r & 7) >> 1, lo = r & 1;
    float v[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int dim = 32 * g16 + 8 * c + s;
      float x = 0.f;
      if (gq < G) {
        if (SQ) {
          if (!rowsig && dim >= 4) x = sgam[dim] * sqr[gq][dim];
        } else if (SPL) {
          // plane 0: outlier beta / regular c_1; plane 1: outlier alpha (chunk 0)
          if (!rowsig && p == 0) x = (c == 0 ? spl_b : spl_c1) * sqr[gq][dim];
          if (!rowsig && p == 1 && c == 0) x = spl_a * sqr[gq][dim];
          if (rowsig && sign_part) x = sqs[gq][dim];
        } else {
          if (!rowsig && !sign_part) x = wp[p] * sqr[gq][dim];
          if (rowsig && sign_part) x = sqs[gq][dim];
        }
      }
      const float hi = f16v(f16b(x));
      v[s] = lo ? x - hi : x;
    }
    u32x4 fr;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) fr[s2] = f16b(v[2 * s2]) | (f16b(v[2 * s2 + 1]) << 16);
    sA[f][lane] = fr;
  }
  __syncthreads();

  // QJL factor sqrt(pi/2)/m; split keys: per group, m_g = 96 (regular) and 32
  const float coef_scale = kQjl / float(SPL ? D - 32 : kc.m);
  const float coef_scale_o = kQjl / 32.f;
  // SQ: the query whose table part this lane forms (see the score step)
  const int q_own = ((g16 & 1) << 1) | (g16 >> 1);
  const float* slow_own = &slow[SQ ? q_own : 0][0][0];
  const float smu_own = SQ ? smu[q_own] : 0.f;
  float sqs_own[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sqs_own[i] = SQ ? sqs[q_own][i] : 0.f;

  // running softmax state of the 2 queries handled by this lane's group (groups 0, 1)
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
  f32x4 accv[8];
#pragma unroll
  for (int vb = 0; vb < 8; ++vb) accv[vb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tiles tile, tile + 4, ... alternate between two register sets (no copies
  // between them, so nothing waits for the next tile's loads early)
  auto process = [&](const TileRegs& R, int tile) {
    uint32_t kw[4][NP], vw[8][2];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (SPL && p == 1) {
        // replicated dword of token 16 g16 + n -> lane (n, g16) gets token
        // 16 nb + n's dword; byte g16 of it holds block g16's 8 outlier bits
        const uint32_t w1 = R.kw4[1][0];
        const u32x4 t = transpose4(u32x4{w1, w1, w1, w1}, lane);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) kw[nb][1] = (t[nb] >> (8 * g16)) & 0xffu;
        continue;
      }
      const u32x4 t = transpose4(R.kw4[p], lane);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) kw[nb][p] = t[nb];  // dword g16 of token 16 nb + n
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 t = transpose4(R.vw4[j], lane);
      vw[2 * j][0] = t[0];
      vw[2 * j][1] = t[1];
      vw[2 * j + 1][0] = t[2];
      vw[2 * j + 1][1] = t[3];
    }
    float nx[4], nr[4], nv[4], nxo[4], nro[4];
    uint32_t sqb[4];  // SQ: plane-0 byte 0 | tail byte << 8 | sign byte << 16
    const uint32_t kpack = R.nx | (R.nr << 16);
    const uint32_t opack = SPL ? (R.xo | (R.ro << 16)) : 0u;
    const uint32_t spack = SQ ? ((R.kw4[0][0] & 0xffu) | (R.tl << 8) | (R.sg << 16)) : 0u;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint32_t kk = uint32_t(__shfl(int(kpack), 16 * nb + n, 64));
      nx[nb] = h2f(uint16_t(kk & 0xffffu));
      nr[nb] = h2f(uint16_t(kk >> 16));
      if (SPL) {
        const uint32_t ko = uint32_t(__shfl(int(opack), 16 * nb + n, 64));
        nxo[nb] = h2f(uint16_t(ko & 0xffffu));
        nro[nb] = h2f(uint16_t(ko >> 16));
      }
      nv[nb] = h2f(uint16_t(__shfl(int(R.nv), 16 * nb + n, 64)));
      sqb[nb] = SQ ? uint32_t(__shfl(int(spack), 16 * nb + n, 64)) : 0u;
    }
    // value B fragments: table lookups issued before the score step
    u32x4 Bv[8][2];
#pragma unroll
    for (int vb = 0; vb < 8; ++vb)
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        const uint32_t w = vw[vb][kc2];
        const uint32_t* lut = slut + (lane & 31);
        Bv[vb][kc2][0] = lut[(w & 0xffu) << 5];
        Bv[vb][kc2][1] = lut[((w >> 8) & 0xffu) << 5];
        Bv[vb][kc2][2] = lut[((w >> 16) & 0xffu) << 5];
        Bv[vb][kc2][3] = lut[(w >> 24) << 5];
      }
    // ---- scores
    float lg[4][2];
    u32x4 A[NP][4];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int c = 0; c < 4; ++c) A[p][c] = sA[p * 4 + c][lane];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 acco = f32x4{0.f, 0.f, 0.f, 0.f};  // split keys: outlier chain
      if (SPL) {
        acco = mfma16(A[0][0], spm[kw[nb][0] & 0xffu], acco);
        acc = mfma16(A[0][1], spm[(kw[nb][0] >> 8) & 0xffu], acc);
        acco = mfma16(A[1][0], spm[kw[nb][1]], acco);
        acc = mfma16(A[0][2], spm[(kw[nb][0] >> 16) & 0xffu], acc);
        acco = mfma16(A[2][0], spm[kw[nb][2] & 0xffu], acco);
        acc = mfma16(A[0][3], spm[kw[nb][0] >> 24], acc);
        acc = mfma16(A[2][1], spm[(kw[nb][2] >> 8) & 0xffu], acc);
        acc = mfma16(A[2][2], spm[(kw[nb][2] >> 16) & 0xffu], acc);
        acc = mfma16(A[2][3], spm[kw[nb][2] >> 24], acc);
      } else {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          acc = mfma16(A[p][0], spm[kw[nb][p] & 0xffu], acc);
          acc = mfma16(A[p][1], spm[(kw[nb][p] >> 8) & 0xffu], acc);
          acc = mfma16(A[p][2], spm[(kw[nb][p] >> 16) & 0xffu], acc);
          acc = mfma16(A[p][3], spm[kw[nb][p] >> 24], acc);
        }
      }
      const float xa = acc[0] + acc[1], xb = acc[2] + acc[3];
      const int tok = tile * kTile + 16 * nb + n;
      const bool valid = tok < len;
      const float coef = nr[nb] * coef_scale;
      float ta, tb;  // score parts beyond the MFMA rows of queries qa = 2 (g16 & 1), qb = qa + 1
      if (SPL) {
        // regular part n_x (code + coef sign) plus the outlier part with its own norms
        const float oa = acco[0] + acco[1], ob = acco[2] + acco[3];
        const float co = nro[nb] * coef_scale_o;
        const float sa = nx[nb] * (xa + coef * xor32(xa, lane)) + nxo[nb] * (oa + co * xor32(oa, lane));
        const float sb = nx[nb] * (xb + coef * xor32(xb, lane)) + nxo[nb] * (ob + co * xor32(ob, lane));
        lg[nb][0] = valid ? a.scale * sa : -INFINITY;
        lg[nb][1] = valid ? a.scale * sb : -INFINITY;
        continue;
      }
      if (SQ) {
        // dims 0..3 from the table, the mu part and the 4 signs, for one query
        // per lane (q_own), the partner query's part from the lane 32 away:
        // lanes (n, 0) / (n, 2) take queries 0 / 1, lanes (n, 1) / (n, 3) 2 / 3
        const uint32_t w = sqb[nb];
        const uint32_t tl = stail[(w >> 8) & 0xffu];
        float e = smu_own;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t idx = ((w >> i) & 1u) | ((tl >> (5 * i)) & 31u);
          e += slow_own[i * kMaxLevels + idx];
          const float sg = (w >> (16 + i)) & 1u ? sqs_own[i] : -sqs_own[i];
          e = fmaf(coef, sg, e);
        }
        ta = e;
        tb = xor32(e, lane);
        if (g16 >= 2) { const float t = ta; ta = tb; tb = t; }
      } else {
        ta = coef * xor32(xa, lane);
        tb = coef * xor32(xb, lane);
      }
      lg[nb][0] = valid ? a.scale * nx[nb] * (xa + ta) : -INFINITY;
      lg[nb][1] = valid ? a.scale * nx[nb] * (xb + tb) : -INFINITY;
    }
    // ---- online softmax (lanes of group 0: queries 0,1; group 1: queries 2,3)
    float alpha[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float mt = fmaxf(fmaxf(lg[0][k], lg[1][k]), fmaxf(lg[2][k], lg[3][k]));
      mt = grp_max<G>(mt);
      const float mnew = fmaxf(mrun[k], mt);
      alpha[k] = mrun[k] == -INFINITY ? 0.f : __expf(mrun[k] - mnew);
      float ps = 0.f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float p = mnew == -INFINITY ? 0.f : __expf(lg[nb][k] - mnew);
        ps += p;
        const int q = 2 * g16 + k;
        if (g16 < 2 && q < G) sP[wave][q][16 * nb + n] = uint16_t(f16b(p * nv[nb]));
      }
      lrun[k] = lrun[k] * alpha[k] + grp_sum(ps);
      mrun[k] = mnew;
    }
    // rescale: accumulator rows = queries 0..3 in lane group 0
    const float al01 = alpha[0], al11 = alpha[1];
    const float al2 = xor16(al01, lane), al3 = xor16(al11, lane);
    __builtin_amdgcn_wave_barrier();
    // ---- P V_hat
    u32x4 Ap[2];
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2)
      Ap[kc2] = *reinterpret_cast<const u32x4*>(&sP[wave][n][32 * kc2 + 8 * g16]);
#pragma unroll
    for (int vb = 0; vb < 8; ++vb) {
      accv[vb][0] *= al01;
      accv[vb][1] *= al11;
      accv[vb][2] *= al2;
      accv[vb][3] *= al3;
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        accv[vb] = mfma16(Ap[kc2], Bv[vb][kc2], accv[vb]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  // the prefetches are unconditional (clamped to the last tile, a harmless
  // re-read) so that the wait counters stay exact across the loop
  for (int tile = t_begin + wave; tile < t_end; tile += 8) {
    load_tile(min(tile + 4, t_end - 1), rb);
    process(ra, tile);
    if (tile + 4 >= t_end) break;
    load_tile(min(tile + 8, t_end - 1), ra);
    process(rb, tile + 4);
  }
  // ---- merge the 4 waves: group-0 lanes hold rows (queries) 0..3 of coord 16vb+n
  if (g16 < 2 && n == 0) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      sm_m[wave][2 * g16 + k] = mrun[k];
      sm_l[wave][2 * g16 + k] = lrun[k];
    }
  }
  if (g16 == 0) {
#pragma unroll
    for (int vb = 0; vb < 8; ++vb)
#pragma unroll
      for (int q = 0; q < 4; ++q) sacc[wave][q][16 * vb + n] = accv[vb][q];
  }
  __syncthreads();
  if (a.nsplit > 1) {
    float* out = a.part + ((int64_t(b) * a.Hkv + g) * a.nsplit + split) * (G * (2 + D));
    for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
      const int gg = e / D, i = e % D;
      float M = -INFINITY;
      for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][gg]);
      float accs = 0.f, l = 0.f;
      for (int w = 0; w < 4; ++w) {
        const float f = sm_m[w][gg] == -INFINITY ? 0.f : __expf(sm_m[w][gg] - M);
        accs += f * sacc[w][gg][i];
        l += f * sm_l[w][gg];
      }
      out[2 * G + gg * D + i] = accs;
      if (i == 0) { out[gg] = M; out[G + gg] = l; }
    }
    return;
  }
  // one split per sequence: normalise and rotate back here,
  // out_i = sum_k Pi_v[k][i] y_k with y = acc / l (the query set-up arrays
  // are free again and hold y and the second half's sums)
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int gg = e / D, i = e % D;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][gg]);
    float accs = 0.f, l = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = sm_m[w][gg] == -INFINITY ? 0.f : __expf(sm_m[w][gg] - M);
      accs += f * sacc[w][gg][i];
      l += f * sm_l[w][gg];
    }
    sqr[gg][i] = l > 0.f ? accs / l : 0.f;
  }
  __syncthreads();
  {
    const int i = threadIdx.x & (D - 1), half = threadIdx.x >> 7;
    const int hv = vc.heads > 1 ? g : 0;
    const float* rot = vc.rot + size_t(hv) * D * D + size_t(64 * half) * D + i;
    float o[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) o[gg] = 0.f;
#pragma unroll
    for (int k0 = 0; k0 < 64; k0 += 16) {
      float r[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) r[u] = rot[size_t(k0 + u) * D];
#pragma unroll
      for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int gg = 0; gg < G; ++gg) o[gg] = fmaf(r[u], sqr[gg][64 * half + k0 + u], o[gg]);
    }
    if (half == 1) {
#pragma unroll
      for (int gg = 0; gg < G; ++gg) sqs[gg][i] = o[gg];
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int gg = 0; gg < G; ++gg)
        a.out[(int64_t(b) * a.Hq + g * G + gg) * D + i] = o[gg] + sqs[gg][i];
    }
  }
}

}  // namespace

// SpectralQuant key codec the MFMA kernel handles: one bit on dims 4..127,
// 1..5 bits on dims 0..3 whose extra bits fit one tail byte, 4 QJL signs.
static bool sq_keys(const CodecView& kv) {
  if (kv.uniform || kv.mode != TQ_PROD || kv.m != 4 || kv.layout != TQ_LAYOUT_ROW) return false;
  if (kv.tail_bits > 8 || kv.code_bytes != 17 - (kv.tail_bits == 0) || kv.sign_bytes != 1) return false;
  return kv.sq_ok != 0;
}

// Outlier-split key codec the MFMA kernel handles: 32 outlier coordinates
// (o4 = 8) with 2 index bits, the rest 1, full block sketch.
static bool split_keys(const CodecView& kv) {
  return kv.outl && kv.o4 == 8 && kv.split_ub_o == 2 && kv.split_ub_r == 1 && kv.mode == TQ_PROD &&
         kv.m == D && kv.code_bytes == 20 && kv.layout == TQ_LAYOUT_ROW;
}

bool decode_mfma_supported(const CodecView& kv, const CodecView& vv, int G) {
  const bool keys = kv.d == D && kv.layout == TQ_LAYOUT_ROW &&
                    ((kv.uniform && kv.mode == TQ_PROD && kv.m == D && (kv.ubits == 1 || kv.ubits == 2)) ||
                     sq_keys(kv) || split_keys(kv));
  return keys && vv.d == D && vv.uniform && vv.mode == TQ_MSE && vv.layout == TQ_LAYOUT_COL &&
         vv.ubits == 4 && (G == 1 || G == 2 || G == 4);
}

hipError_t launch_decode_mfma(const CodecView& kv, const CodecView& vv, const DecodeArgs& a,
                              hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  dim3 grid(unsigned(a.nsplit), unsigned(a.Hkv), unsigned(a.B));
#define TQ_LAUNCH(GG, UU) hipLaunchKernelGGL((decode_mfma_kernel<GG, UU>), grid, dim3(256), 0, s, kv, vv, a)
  if (kv.outl) {
    if (G == 4) TQ_LAUNCH(4, 3); else if (G == 2) TQ_LAUNCH(2, 3); else TQ_LAUNCH(1, 3);
  } else if (!kv.uniform) {
    if (G == 4) TQ_LAUNCH(4, 0); else if (G == 2) TQ_LAUNCH(2, 0); else TQ_LAUNCH(1, 0);
  } else if (kv.ubits == 2) {
    if (G == 4) TQ_LAUNCH(4, 2); else if (G == 2) TQ_LAUNCH(2, 2); else TQ_LAUNCH(1, 2);
  } else {
    if (G == 4) TQ_LAUNCH(4, 1); else if (G == 2) TQ_LAUNCH(2, 1); else TQ_LAUNCH(1, 1);
  }
#undef TQ_LAUNCH
  return hipGetLastError();
}

}  // namespace tq
