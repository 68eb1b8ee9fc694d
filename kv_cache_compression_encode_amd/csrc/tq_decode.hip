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
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr float kQjl = 1.2533141373155001f;  // sqrt(pi / 2)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x for x <= 0 (or -inf): the hardware base-2 exponential
__device__ __forceinline__ float exp2_le0(float x) { return __builtin_amdgcn_exp2f(x); }

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
// (a row rotation reads a valid lane everywhere, so the move needs no old
// value and the compiler folds it into the max or add as a DPP operand)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
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

// NW waves per workgroup: 4 (two workgroups per CU), or 8 (one per CU, for
// small batches split into many workgroups: the set-up, which loads the
// columns of Pi and S, then runs once per CU)
// VK: the value records.  0: TurboQuant-mse col records with 4 index bits.
// 1: 2.5-bit outlier-split mse values in col records: for each 8-token group
// the 16 lane blocks (block n: coordinates 16 vb + n, vb = 0..7; 3-byte slots
// of 3-bit codes for the outlier coordinates, vb even and n < 8, 2-byte slots
// of 2-bit codes otherwise), 288 bytes a group, then the two groups' norms.
// Lane (n, g16) loads its block of token groups g16 and 4 + g16, which hold
// exactly its B operands; each token pair's codes index a 2-token LUT of its
// group (16 regular, 64 outlier entries) and the pair's group norms are
// multiplied in, so P carries the softmax weights alone.
template <int G, int UB, int NW, int VK = 0>
__global__ __launch_bounds__(64 * NW, 8 / NW) void decode_mfma_kernel(CodecView kc, CodecView vc, DecodeArgs a) {
  static_assert(G >= 1 && G <= 4, "up to 4 query heads per KV head");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int NT = 64 * NW;  // threads
  constexpr bool SQ = UB == 0;
  constexpr bool SPL = UB == 3;  // outlier-channel split keys, 32 outlier coordinates
  __shared__ __align__(16) float sqr[4][D];
  __shared__ __align__(16) float sqs[4][D];
  // SQ, per query: [i][idx] = q'_i c_i(idx) for dims i = 0..3, and [4][s] =
  // sum_i (+-qs_i) over the 4 QJL sign bits s (bit set: +).  Query q's tables
  // start at 336 q words: queries 0 and 2 (1 and 3), whose lanes read in the
  // same LDS cycle, then sit 32 banks apart
  constexpr int kSqtab = 336;
  __shared__ float sqtab[SQ ? 4 * kSqtab : 1];
  __shared__ float smu[4];
  __shared__ __align__(16) float sgam[SQ ? D : 1];
  __shared__ float smuv[SQ ? D : 1];  // SQ: one-bit dims' (c1 - c0)/2, (c1 + c0)/2
  // SQ: tail byte -> byte i = 4 x (index bits 1.. of dim i), i = 0..3: with
  // the low bits added, byte i is the byte offset of dim i's table entry
  __shared__ uint32_t stail[SQ ? 256 : 1];
  __shared__ float skc[SQ ? 4 : 1][kMaxLevels];  // SQ: levels of dims 0..3
  // value byte (two 4-bit codes) -> fp16 pair of their levels, 32 copies:
  // entry e for lane l at slut[e * 32 + l % 32], so that the random lookups
  // of a wave hit 32 distinct banks
  __shared__ uint32_t slut1[256];
  __shared__ __align__(16) uint32_t slut[256 * 32];
  constexpr int PROW = 64 + 8;  // padded row of the P buffer (bank spread)
  __shared__ __align__(16) uint16_t sP[NW][16][PROW];  // per wave: [query row][token] fp16 weights
  __shared__ float sm_m[NW][4], sm_l[NW][4];
  __shared__ float sacc[NW][4][D];

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
    uint32_t vcw[2][5];   // VK 1: the lane block of token groups g16, 4 + g16
    u32x4 vnr[2], vno[2];  // VK 1: fp16 norm pairs of those tokens (regular, outlier)
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
    if constexpr (VK == 0) {
      // load j: dim 16 (2j + g16/2) + n, bytes 16 (g16 % 2) .. + 15 of its field
#pragma unroll
      for (int j = 0; j < 4; ++j)
        R.vw4[j] = *reinterpret_cast<const u32x4*>(vt + (16 * (2 * j + (g16 >> 1)) + n) * 32 + 16 * (g16 & 1));
      R.nv = *reinterpret_cast<const uint16_t*>(vt + vc.off_nx + 2 * tok);
    } else {
      const int boff = n < 8 ? 20 * n : 160 + 16 * (n - 8);
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        const uint32_t* blk = reinterpret_cast<const uint32_t*>(vt + (4 * kc2 + g16) * 288 + boff);
#pragma unroll
        for (int u = 0; u < 5; ++u) R.vcw[kc2][u] = blk[u];  // the fifth word of an n >= 8 block goes unused
        R.vnr[kc2] = *reinterpret_cast<const u32x4*>(vt + vc.off_nx + 2 * (32 * kc2 + 8 * g16));
        R.vno[kc2] = *reinterpret_cast<const u32x4*>(vt + vc.off_nxo + 2 * (32 * kc2 + 8 * g16));
      }
      R.nv = 0x3C00u;  // 1.0: the norms are in the B operand
    }
    R.nx = *reinterpret_cast<const uint16_t*>(kt + kc.off_nx + 2 * tok);
    R.nr = *reinterpret_cast<const uint16_t*>(kt + kc.off_nr + 2 * tok);
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
  // the raw queries are loaded first (512 values over the threads; their
  // latency is the first the set-up waits for)
  constexpr int QPT = 4 * D / NT;
  float qraw[QPT];
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int e = threadIdx.x + NT * u;
    const int gg = e / D, i = e % D;
    const int64_t qi = int64_t(b) * a.Hq + g * G + gg;
    float v = 0.f;
    if (gg < G)
      v = a.q_bf16 ? __uint_as_float(uint32_t(static_cast<const uint16_t*>(a.q)[qi * D + i]) << 16)
                   : static_cast<const float*>(a.q)[qi * D + i];
    qraw[u] = v;
  }
  // the first tile's loads go out before the set-up below and overlap it.
  // Contiguous records: they do not wait for seq_lens, since any tile below
  // max_tokens is in the records (a wave without a tile leaves them unused).
  // Paged records: only tiles below seq_lens are looked up in the block table
  // (the entries past them need not name pages).
  if (!a.block_table) {
    const int tmax = (a.max_tokens + kTile - 1) / kTile;
    if (tmax > 0) load_tile(min(t_begin + wave, tmax - 1), ra);
  } else if (t_begin + wave < t_end) {
    load_tile(t_begin + wave, ra);
  }

  // ---- set-up: one round of independent loads, then arithmetic on LDS.
  // The G queries are rotated here, q' = Pi_h q and qs = S q'[0:m]: thread t
  // forms coordinate t % 128 over half t / 128 of each sum, reading the
  // transposed matrices column-coalesced (all their loads go out first).
  const int hk = kc.heads > 1 ? g : 0;
  // randomized Hadamard keys: q' = H (s q) / sqrt(d) by the wave transform
  // instead of the columns of Pi
  const bool khad = kc.had_sign != nullptr;
  // thread t takes columns 4 cg .. 4 cg + 3 (cg = t % 32) over the RPT rows
  // RPT rg .. RPT rg + RPT - 1 (rg = t / 32) of the transposed matrices, as
  // 16-byte loads; the NRG row groups' partial sums are added through LDS
  constexpr int NRG = NT / 32, RPT = D / NRG;
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  float4 rc4[RPT], sc4[RPT];  // sc4 unused (never loaded) for SpectralQuant keys
  {
    const float* rt = kc.rot_t + size_t(hk) * D * D + size_t(RPT * rg) * D + 4 * cg;
    if (!khad) {
#pragma unroll
      for (int u = 0; u < RPT; ++u) rc4[u] = *reinterpret_cast<const float4*>(rt + size_t(u) * D);
    }
    if (!SQ) {
      const float* st = kc.sketch_t + size_t(RPT * rg) * D + 4 * cg;
#pragma unroll
      for (int u = 0; u < RPT; ++u) sc4[u] = *reinterpret_cast<const float4*>(st + size_t(u) * D);
    }
  }
#pragma unroll
  for (int u = 0; u < QPT; ++u) (&sqs[0][0])[threadIdx.x + NT * u] = qraw[u];  // raw queries, staged in sqs
  const float* kcen = kc.cen + size_t(hk) * D * kMaxLevels;
  if (threadIdx.x < 256) {
    const int t = threadIdx.x;  // one value-table entry per thread
    if constexpr (VK == 0) {
      slut1[t] = f16b(vc.ucen[t & 15]) | (f16b(vc.ucen[t >> 4]) << 16);
    } else {
      // entries 0..15: regular token pairs (i0 | i1 << 2, levels of stored
      // dim 8); 16..79: outlier pairs (i0 | i1 << 3, levels of stored dim 0)
      const float* ce = vc.cen + size_t(vc.heads > 1 ? g : 0) * D * kMaxLevels;
      uint32_t v = 0u;
      if (t < 16) v = f16b(ce[8 * kMaxLevels + (t & 3)]) | (f16b(ce[8 * kMaxLevels + (t >> 2)]) << 16);
      else if (t < 80) v = f16b(ce[(t - 16) & 7]) | (f16b(ce[(t - 16) >> 3]) << 16);
      slut1[t] = v;
    }
  }
  for (int e = threadIdx.x; e < NW * 16 * PROW / 8; e += blockDim.x)
    reinterpret_cast<u32x4*>(&sP[0][0][0])[e] = u32x4{0u, 0u, 0u, 0u};
  if (SQ && threadIdx.x < 256) {
    {
      const uint32_t tw = kc.sq_tail[threadIdx.x];  // dim i's bits 1.. at bits 5i .. 5i + 4
      uint32_t b = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) b |= (((tw >> (5 * i)) & 31u) << 2) << (8 * i);
      stail[threadIdx.x] = b;
    }
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
    // q' = Pi q: row-group partial sums into the (not yet filled) value
    // table, then added
    float* part = reinterpret_cast<float*>(slut);  // [NRG][4][D]
    static_assert(NRG * 4 * D <= 256 * 32, "partials fit the value table");
    // partial sums of the 4 queries over this thread's rows, 4 columns each
    auto rowgroup = [&](const float4 (&m4)[RPT], const float (&x)[4][D]) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
          const float xv = x[gg][RPT * rg + u];
          acc.x = fmaf(m4[u].x, xv, acc.x);
          acc.y = fmaf(m4[u].y, xv, acc.y);
          acc.z = fmaf(m4[u].z, xv, acc.z);
          acc.w = fmaf(m4[u].w, xv, acc.w);
        }
        *reinterpret_cast<float4*>(&part[(rg * 4 + gg) * D + 4 * cg]) = acc;
      }
    };
    auto gather = [&](float (&y)[4][D]) {
      for (int e = threadIdx.x; e < 4 * D; e += blockDim.x) {
        float v = 0.f;
#pragma unroll
        for (int r8 = 0; r8 < NRG; ++r8) v += part[r8 * 4 * D + e];
        y[e / D][e % D] = v;
      }
    };
    if (khad) {
      // wave w < 4 transforms query w
      if (wave < 4) {
        float lo = sqs[wave][lane] * kc.had_sign[lane], hi = sqs[wave][lane + 64] * kc.had_sign[lane + 64];
        fwht128_wave(lo, hi, lane);
        sqr[wave][lane] = lo * kInvSqrt128;
        sqr[wave][lane + 64] = hi * kInvSqrt128;
      }
    } else {
      rowgroup(rc4, sqs);
      __syncthreads();
      gather(sqr);
    }
    __syncthreads();
    if (!SQ) {
      // qs = S q' (m = d)
      rowgroup(sc4, sqr);
      __syncthreads();
      gather(sqs);
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
#pragma unroll
  for (int k = 0; k < 2048 / NT; ++k) {  // consecutive threads write consecutive 16-byte groups
    const int e4 = k * NT + threadIdx.x;
    const uint32_t v = slut1[e4 >> 3];
    reinterpret_cast<u32x4*>(slut)[e4] = u32x4{v, v, v, v};
  }
  if (SQ) {
    for (int e = threadIdx.x; e < 4 * 4 * kMaxLevels; e += blockDim.x) {
      const int gg = e / (4 * kMaxLevels), i = (e / kMaxLevels) % 4, l = e % kMaxLevels;
      sqtab[gg * kSqtab + i * 64 + l] = sqr[gg][i] * skc[i][l];
    }
    if (threadIdx.x < 64) {
      const int gg = threadIdx.x >> 4, sb = threadIdx.x & 15;
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) v += ((sb >> i) & 1) ? sqs[gg][i] : -sqs[gg][i];
      sqtab[gg * kSqtab + 4 * 64 + sb] = v;
    }
    if (wave < 4) {  // wave w: sum_{i >= 4} mu_i q'_i of query w
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
  if (threadIdx.x < 256) {
    const uint32_t e = threadIdx.x;
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = (((e >> (2 * j)) & 1u) ? 0x3C00u : 0xBC00u) | ((((e >> (2 * j + 1)) & 1u) ? 0x3C00u : 0xBC00u) << 16);
    spm[e] = r;
  }
  for (int f = wave; f < NP * 4; f += NW) {
    const int p = f / 4, c = f % 4;
    const bool sign_part = p == NP - 1;
    const int r = n;
    const bool rowsig = r >= 8;
    const int gq = (r & 7) >> 1, lo = r & 1;
    const int dim0 = 32 * g16 + 8 * c;
    // the 8 consecutive dims of this lane, two 16-byte reads each
    float qv[8], gv[8];
    {
      const float* src = (rowsig ? &sqs[gq & 3][0] : &sqr[gq & 3][0]) + dim0;
      const float4 u0 = *reinterpret_cast<const float4*>(src), u1 = *reinterpret_cast<const float4*>(src + 4);
      qv[0] = u0.x; qv[1] = u0.y; qv[2] = u0.z; qv[3] = u0.w;
      qv[4] = u1.x; qv[5] = u1.y; qv[6] = u1.z; qv[7] = u1.w;
      if (SQ) {
        const float4 w0 = *reinterpret_cast<const float4*>(&sgam[dim0]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sgam[dim0 + 4]);
        gv[0] = w0.x; gv[1] = w0.y; gv[2] = w0.z; gv[3] = w0.w;
        gv[4] = w1.x; gv[5] = w1.y; gv[6] = w1.z; gv[7] = w1.w;
      }
    }
    float v[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int dim = dim0 + s;
      float x = 0.f;
      if (gq < G) {
        if (SQ) {
          if (!rowsig && dim >= 4) x = gv[s] * qv[s];
        } else if (SPL) {
          // plane 0: outlier beta / regular c_1; plane 1: outlier alpha (chunk 0)
          if (!rowsig && p == 0) x = (c == 0 ? spl_b : spl_c1) * qv[s];
          if (!rowsig && p == 1 && c == 0) x = spl_a * qv[s];
          if (rowsig && sign_part) x = qv[s];
        } else {
          if (!rowsig && !sign_part) x = wp[p] * qv[s];
          if (rowsig && sign_part) x = qv[s];
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

  // logits in base-2 units (softmax scale times log2 e), so that each
  // exponential is one v_exp_f32; the running maxima are in the same units
  // and go back to natural units only where partials leave the kernel
  const float scale2 = a.scale * kLog2e;
  // QJL factor sqrt(pi/2)/m; split keys: per group, m_g = 96 (regular) and 32
  const float coef_scale = kQjl / float(SPL ? D - 32 : kc.m);
  const float coef_scale_o = kQjl / 32.f;
  // SQ: the query whose table part this lane forms (see the score step)
  const int q_own = ((g16 & 1) << 1) | (g16 >> 1);
  // byte offset of this query's tables in sqtab
  const uint32_t qtab = SQ ? uint32_t(q_own) * (kSqtab * 4) : 0u;
  const char* sqtab_b = reinterpret_cast<const char*>(&sqtab[0]);
  const float smu_own = SQ ? smu[q_own] : 0.f;

  // running softmax state of the 2 queries handled by this lane's group (groups 0, 1)
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
  f32x4 accv[8];
#pragma unroll
  for (int vb = 0; vb < 8; ++vb) accv[vb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tiles tile, tile + NW, ... alternate between two register sets (no copies
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
    if constexpr (VK == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 t = transpose4(R.vw4[j], lane);
        vw[2 * j][0] = t[0];
        vw[2 * j][1] = t[1];
        vw[2 * j + 1][0] = t[2];
        vw[2 * j + 1][1] = t[3];
      }
    }
    float nx[4], nr[4], nv[4], nxo[4], nro[4];
    // SQ, per token before the exchange (once per token instead of once per
    // token and query): the byte offsets 4 idx_i of dims 0..3 in their tables
    // (low index bits = plane-0 bits 0..3, spread to bit 2 of each byte), and
    // the sign-table offset 4 s in byte 2 of the n_v word
    uint32_t sqb[4], nvb[4];
    const uint32_t kpack = R.nx | (R.nr << 16);
    const uint32_t opack = SPL ? (R.xo | (R.ro << 16)) : 0u;
    const uint32_t spack = SQ ? ((((R.kw4[0][0] & 0xfu) * 0x810204u) & 0x04040404u) | stail[R.tl]) : 0u;
    const uint32_t nvpack = SQ ? (R.nv | ((R.sg & 0xfu) << 18)) : R.nv;
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
      nvb[nb] = uint32_t(__shfl(int(nvpack), 16 * nb + n, 64));
      nv[nb] = h2f(uint16_t(nvb[nb] & 0xffffu));
      sqb[nb] = SQ ? uint32_t(__shfl(int(spack), 16 * nb + n, 64)) : 0u;
    }
    // ---- scores: the four 16-key blocks accumulate in four independent
    // MFMA chains, interleaved step by step (each chain's next MFMA is four
    // MFMAs away, past its predecessor's latency); the operands of step k + 1
    // (one query fragment, four key patterns) are read during step k
    float lg[4][2];
    constexpr int KPN = SPL ? 9 : NP * 4;  // score MFMAs per 16 keys
    // split keys: step k's (plane, byte) and whether it feeds the outlier chain
    constexpr int spl_p[9] = {0, 0, 1, 0, 2, 0, 2, 2, 2};
    constexpr int spl_c[9] = {0, 1, 0, 2, 0, 3, 1, 2, 3};
    constexpr bool spl_o[9] = {true, false, true, false, true, false, false, false, false};
    auto kbyte = [&](int nb, int k) -> uint32_t {
      if constexpr (SPL) return spl_p[k] == 1 ? kw[nb][1] : (kw[nb][spl_p[k]] >> (8 * spl_c[k])) & 0xffu;
      else return (kw[nb][k >> 2] >> (8 * (k & 3))) & 0xffu;
    };
    auto afrag = [&](int k) -> u32x4 { return SPL ? sA[spl_p[k] * 4 + spl_c[k]][lane] : sA[k][lane]; };
    f32x4 accs[4], accso[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      accs[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      accso[nb] = f32x4{0.f, 0.f, 0.f, 0.f};  // split keys: outlier chain
    }
    u32x4 Ak[2], Bk[2][4];
    Ak[0] = afrag(0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) Bk[0][nb] = spm[kbyte(nb, 0)];
#pragma unroll
    for (int k = 0; k < KPN; ++k) {
      if (k + 1 < KPN) {
        Ak[(k + 1) & 1] = afrag(k + 1);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) Bk[(k + 1) & 1][nb] = spm[kbyte(nb, k + 1)];
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        if (SPL && spl_o[k]) accso[nb] = mfma16(Ak[k & 1], Bk[k & 1][nb], accso[nb]);
        else accs[nb] = mfma16(Ak[k & 1], Bk[k & 1][nb], accs[nb]);
      }
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const f32x4 acc = accs[nb], acco = accso[nb];
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
        lg[nb][0] = valid ? scale2 * sa : -INFINITY;
        lg[nb][1] = valid ? scale2 * sb : -INFINITY;
        continue;
      }
      if (SQ) {
        // dims 0..3 from the table, the mu part and the 4 signs, for one query
        // per lane (q_own), the partner query's part from the lane 32 away:
        // lanes (n, 0) / (n, 2) take queries 0 / 1, lanes (n, 1) / (n, 3) 2 / 3
        const uint32_t w = sqb[nb];
        float e = smu_own;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          e += *reinterpret_cast<const float*>(sqtab_b + 256 * i + (qtab + ((w >> (8 * i)) & 0xffu)));
        e = fmaf(coef, *reinterpret_cast<const float*>(sqtab_b + 1024 + (qtab + ((nvb[nb] >> 16) & 0xffu))), e);
        ta = e;
        tb = xor32(e, lane);
        if (g16 >= 2) { const float t = ta; ta = tb; tb = t; }
      } else {
        ta = coef * xor32(xa, lane);
        tb = coef * xor32(xb, lane);
      }
      lg[nb][0] = valid ? scale2 * nx[nb] * (xa + ta) : -INFINITY;
      lg[nb][1] = valid ? scale2 * nx[nb] * (xb + tb) : -INFINITY;
    }
    // value B fragments: table lookups issued before the softmax, whose
    // arithmetic covers their latency
    u32x4 Bv[8][2];
    if constexpr (VK == 0) {
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
    } else {
      // slot vb of the lane block: bytes 5 (vb / 2) + 3 (vb % 2) (n < 8) or
      // 2 vb (n >= 8); 3-bit codes in the outlier slots (n < 8, vb even)
      const bool lo8 = n < 8;
      const uint32_t* lut = slut + (lane & 31);
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        uint32_t c[6];
#pragma unroll
        for (int u = 0; u < 5; ++u) c[u] = R.vcw[kc2][u];
        c[5] = 0u;
#pragma unroll
        for (int vb = 0; vb < 8; ++vb) {
          const int obo = 5 * (vb >> 1) + 3 * (vb & 1), obr = 2 * vb;
          const uint32_t wo = __builtin_amdgcn_alignbyte(c[obo / 4 + 1], c[obo / 4], obo % 4);
          const uint32_t wr = __builtin_amdgcn_alignbyte(c[obr / 4 + 1], c[obr / 4], obr % 4);
          const bool three = lo8 && !(vb & 1);
          const uint32_t w = lo8 ? wo : wr;
          const uint32_t bs2 = three ? 6u : 4u;       // bits per token pair
          const uint32_t base = three ? (16u << 5) : 0u;
          // the norm words go through scalars: a bit cast straight from a
          // vector element has read element 0
          uint32_t nw[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) nw[k] = three ? R.vno[kc2][k] : R.vnr[kc2][k];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t e = __builtin_amdgcn_ubfe(w, bs2 * k, bs2);
            const uint32_t lv = lut[base + (e << 5)];
            const uint32_t nk = nw[k];
            const h2_t prod = __builtin_bit_cast(h2_t, lv) * __builtin_bit_cast(h2_t, nk);
            Bv[vb][kc2][k] = __builtin_bit_cast(uint32_t, prod);
          }
        }
      }
    }
    // ---- online softmax (lanes of group 0: queries 0,1; group 1: queries 2,3)
    float alpha[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float mt = fmaxf(fmaxf(lg[0][k], lg[1][k]), fmaxf(lg[2][k], lg[3][k]));
      mt = grp_max<G>(mt);
      const float mnew = fmaxf(mrun[k], mt);
      alpha[k] = mrun[k] == -INFINITY ? 0.f : exp2_le0(mrun[k] - mnew);
      // no token yet (mnew = -inf): every lg is -inf and exp(lg - 0) = 0
      const float msafe = mnew == -INFINITY ? 0.f : mnew;
      float ps = 0.f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float p = exp2_le0(lg[nb][k] - msafe);
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
    // the accumulators are rescaled only when some query's running maximum
    // moved (a factor of exactly 1 elsewhere), which after the first tiles
    // is the exception
    if (__ballot(al01 != 1.f || al11 != 1.f) != 0) {
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) {
        accv[vb][0] *= al01;
        accv[vb][1] *= al11;
        accv[vb][2] *= al2;
        accv[vb][3] *= al3;
      }
    }
    // the two k-halves as two rounds over the 8 accumulators, so that
    // consecutive MFMAs are independent
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) accv[vb] = mfma16(Ap[kc2], Bv[vb][kc2], accv[vb]);
    __builtin_amdgcn_wave_barrier();
  };
  // the prefetches are unconditional (clamped to the last tile, a harmless
  // re-read) so that the wait counters stay exact across the loop
  for (int tile = t_begin + wave; tile < t_end; tile += 2 * NW) {
    load_tile(min(tile + NW, t_end - 1), rb);
    process(ra, tile);
    if (tile + NW >= t_end) break;
    load_tile(min(tile + 2 * NW, t_end - 1), ra);
    process(rb, tile + NW);
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
  // partials for decode_combine (the 8-wave form is only launched with
  // several splits per sequence)
  if (NW == 8 || a.nsplit > 1) {
    float* out = a.part + ((int64_t(b) * a.Hkv + g) * a.nsplit + split) * (G * (2 + D));
    for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
      const int gg = e / D, i = e % D;
      float M = -INFINITY;
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][gg]);
      float accs = 0.f, l = 0.f;
      for (int w = 0; w < NW; ++w) {
        const float f = sm_m[w][gg] == -INFINITY ? 0.f : exp2_le0(sm_m[w][gg] - M);
        accs += f * sacc[w][gg][i];
        l += f * sm_l[w][gg];
      }
      out[2 * G + gg * D + i] = accs;
      if (i == 0) { out[gg] = M * kLn2; out[G + gg] = l; }  // the maximum in natural units
    }
    return;
  }
  if constexpr (NW == 4) {
  // one split per sequence: normalise and rotate back here,
  // out_i = sum_k Pi_v[k][i] y_k with y = acc / l (the query set-up arrays
  // are free again and hold y and the second half's sums)
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int gg = e / D, i = e % D;
    float M = -INFINITY;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][gg]);
    float accs = 0.f, l = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float f = sm_m[w][gg] == -INFINITY ? 0.f : exp2_le0(sm_m[w][gg] - M);
      accs += f * sacc[w][gg][i];
      l += f * sm_l[w][gg];
    }
    sqr[gg][i] = l > 0.f ? accs / l : 0.f;
  }
  __syncthreads();
  if (vc.had_sign) {
    // randomized Hadamard values: out = s (H y) / sqrt(d), wave w for query w
    if (wave < G) {
      float lo = sqr[wave][lane], hi = sqr[wave][lane + 64];
      fwht128_wave(lo, hi, lane);
      float* o = a.out + (int64_t(b) * a.Hq + g * G + wave) * D;
      o[lane] = vc.had_sign[lane] * lo * kInvSqrt128;
      o[lane + 64] = vc.had_sign[lane + 64] * hi * kInvSqrt128;
    }
    return;
  }
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
  // values: 4-bit col records, or the 2.5-bit split in col records (with split
  // keys or 2-bit TurboQuant-prod keys)
  const bool sv = vv.outl && vv.mode == TQ_MSE && vv.layout == TQ_LAYOUT_COL && vv.o4 == 8 &&
                  vv.split_ub_o == 3 && vv.split_ub_r == 2 &&
                  (split_keys(kv) || (kv.uniform && kv.mode == TQ_PROD && kv.m == D && kv.ubits == 2));
  const bool v4 = vv.uniform && vv.mode == TQ_MSE && vv.layout == TQ_LAYOUT_COL && vv.ubits == 4;
  return keys && vv.d == D && (v4 || sv) && (G == 1 || G == 2 || G == 4);
}

hipError_t launch_decode_mfma(const CodecView& kv, const CodecView& vv, const DecodeArgs& a,
                              hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (a.waves == 8 && a.nsplit < 2) return hipErrorInvalidValue;  // the 8-wave form writes partials only
  dim3 grid(unsigned(a.nsplit), unsigned(a.Hkv), unsigned(a.B));
#define TQ_LAUNCH(GG, UU)                                                                        \
  do {                                                                                            \
    if (a.waves == 8)                                                                             \
      hipLaunchKernelGGL((decode_mfma_kernel<GG, UU, 8>), grid, dim3(512), 0, s, kv, vv, a);      \
    else                                                                                          \
      hipLaunchKernelGGL((decode_mfma_kernel<GG, UU, 4>), grid, dim3(256), 0, s, kv, vv, a);      \
  } while (0)
#define TQ_LAUNCH_SV(GG, UU)                                                                     \
  do {                                                                                            \
    if (a.waves == 8)                                                                             \
      hipLaunchKernelGGL((decode_mfma_kernel<GG, UU, 8, 1>), grid, dim3(512), 0, s, kv, vv, a);   \
    else                                                                                          \
      hipLaunchKernelGGL((decode_mfma_kernel<GG, UU, 4, 1>), grid, dim3(256), 0, s, kv, vv, a);   \
  } while (0)
  if (vv.outl) {
    // split values: split keys or 2-bit TurboQuant-prod keys
    if (kv.outl) {
      if (G == 4) TQ_LAUNCH_SV(4, 3); else if (G == 2) TQ_LAUNCH_SV(2, 3); else TQ_LAUNCH_SV(1, 3);
    } else {
      if (G == 4) TQ_LAUNCH_SV(4, 2); else if (G == 2) TQ_LAUNCH_SV(2, 2); else TQ_LAUNCH_SV(1, 2);
    }
  } else if (kv.outl) {
    if (G == 4) TQ_LAUNCH(4, 3); else if (G == 2) TQ_LAUNCH(2, 3); else TQ_LAUNCH(1, 3);
  } else if (!kv.uniform) {
    if (G == 4) TQ_LAUNCH(4, 0); else if (G == 2) TQ_LAUNCH(2, 0); else TQ_LAUNCH(1, 0);
  } else if (kv.ubits == 2) {
    if (G == 4) TQ_LAUNCH(4, 2); else if (G == 2) TQ_LAUNCH(2, 2); else TQ_LAUNCH(1, 2);
  } else {
    if (G == 4) TQ_LAUNCH(4, 1); else if (G == 2) TQ_LAUNCH(2, 1); else TQ_LAUNCH(1, 1);
  }
#undef TQ_LAUNCH
#undef TQ_LAUNCH_SV
  return hipGetLastError();
}

}  // namespace tq
