// TurboQuant encode, query preparation, scoring and top-k search for rows
// whose dimension d is a multiple of 128 (the 1536-dim vector-search width),
// hand-written for CDNA4 matrix cores.
//
// Every product here has the same shape: a shared operand A (the rotation Pi,
// the sketch S, or a block of 128 queries) staged through LDS in tiles of 32
// reduction elements, against lane-owned rows B (input vectors, residuals, or
// compressed records) that each wave reads straight from memory into MFMA
// operand registers.  A workgroup is 4 waves; a wave owns 64 B rows (two
// 32-row blocks) and computes all 128 A rows for them with
// v_mfma_f32_32x32x16_f16, so its accumulator is 4 x 2 blocks of 32 x 32.
// Within a tile, lane half h supplies reduction elements 16h .. 16h + 15 to
// both operands (8 per MFMA step), so every lane reads 16 consecutive
// elements of its row.
//
// The steps (TurboQuant paper review, "Method"):
//   rowscale : n_x = ||x|| and a power-of-two scale putting max |x_i| in
//              [2^14, 2^15) for the fp16 hi/lo split;
//   rotate   : y = Pi x with fp32 accuracy from fp16 parts (16 Pi = P_hi +
//              P_lo built once with the codebook, x 2^e = X_hi + X_lo split in
//              registers): P_hi X_hi + P_lo X_hi + P_hi X_lo.  The epilogue
//              quantizes each coordinate against the Lloyd-Max boundaries
//              (scaled by the vector's factor instead of dividing y), packs
//              the row-layout bit planes of its 128 coordinates (one 16-byte
//              record chunk per plane), and for prod writes the residual
//              r = y - c[idx] as fp16 hi/lo parts of 2^13 r and the partial
//              sums of ||r||^2;
//   sketch   : z = S r on the residual parts (S is stored exactly in fp16, so
//              S R_hi + S R_lo), sign bits [z >= 0] packed into the record's
//              sign chunks, n_r = ||r||;
//   search   : s = n_x (sum_i q'_i c[idx_i] + n_r sqrt(pi/2)/m sum_j qs_j
//              (2 bit_j - 1)) for 128 queries per workgroup against the
//              records, the key operand built from the record bytes through
//              LDS tables (+-1 patterns for signs and one-bit codes, whose
//              centroid is folded into the query operand; fp16 centroids for
//              2 and 3 index bits), n_r applied between the sign and code
//              phases, n_x in the epilogue; then either the scores are stored
//              or each query's top-k is kept in registers of the lane that
//              owns the query (the paper review's "Results": vector search
//              over the codes) and only the lists leave the chip.
// The rotation and the sketch follow the query preparation q' = Pi q,
// qs = S q' the same way, with fp32 outputs.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "tq_kernels.h"

namespace tq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;

constexpr int NT = 256;        // threads per workgroup (4 waves)
constexpr int KT = 32;         // reduction elements per staged tile
constexpr int AR = 128;        // shared-operand rows per workgroup
constexpr int AP = 40;         // LDS pitch of a staged row in halves: 80 bytes,
                               // so 8 lanes reading 16 bytes of 8 rows hit 32 banks
constexpr int BW = 256;        // lane-owned rows per workgroup (64 per wave)
constexpr float kQjl = 1.2533141373155001f;  // sqrt(pi / 2)
constexpr float kRScale = 8192.f;            // residuals are handed over as 2^13 r

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t h16(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ __forceinline__ float f16f(uint32_t h) { return float(__builtin_bit_cast(_Float16, uint16_t(h))); }

// 8 floats -> fp16 hi (round toward zero) and lo (the exact remainder,
// rounded to nearest): v = hi + lo to about 2^-22 relative.  Each half of a
// lo word is one mixed-precision FMA, v - hi with the fp16 half of hi read in
// place, written straight into its half of the word (mixlo, then mixhi).
__device__ __forceinline__ void split8(const float (&v)[8], u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(v[2 * i], v[2 * i + 1]));
    uint32_t l;
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %1, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(l)
        : "v"(h), "v"(v[2 * i]), "v"(v[2 * i + 1]));
    hi[i] = h;
    lo[i] = l;
  }
}

// Staging of one A tile: NPL planes of [128 rows][32 elements] fp16, stored
// contiguously in global memory (the codebook's tile arrays and the query
// tiles are written in this order), copied to LDS rows of AP halves.
template <int NPL>
struct AStage {
  static constexpr int N = NPL * AR * KT / 8 / NT;  // 16-byte chunks per thread
  u32x4 v[N];
  __device__ __forceinline__ void load(const uint16_t* g) {
#pragma unroll
    for (int u = 0; u < N; ++u) v[u] = reinterpret_cast<const u32x4*>(g)[u * NT + threadIdx.x];
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int e = u * NT + threadIdx.x;
      const int pl = e / (AR * KT / 8), rem = e % (AR * KT / 8);
      const int row = rem / (KT / 8), c8 = rem % (KT / 8);
      *reinterpret_cast<u32x4*>(lds + (pl * AR + row) * AP + c8 * 8) = v[u];
    }
  }
};

// A fragment of MFMA step s of the tile: row 32 c + lane % 32, elements
// 16 (lane / 32) + 8 s .. + 7.
__device__ __forceinline__ u32x4 afrag(const uint16_t* lds, int pl, int c, int s, int lane) {
  return *reinterpret_cast<const u32x4*>(lds + (pl * AR + 32 * c + (lane & 31)) * AP + 16 * (lane >> 5) + 8 * s);
}

// Workgroup -> (row tile, column block), keeping the column blocks of a row
// tile on one XCD (workgroups are dispatched to the 8 XCDs round-robin), so
// that the rows they all read are fetched into that XCD's L2 once.
__device__ __forceinline__ bool map_tile(int nrt, int ncb, int& rt, int& cb) {
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  rt = (j / ncb) * 8 + xcd;
  cb = j % ncb;
  return rt < nrt;
}

// ------------------------------------------------------------- rowscale
// One wave per row: nx = ||x||, sc = 2^e with max |x_i| 2^e in [2^14, 2^15)
// (the squares are summed over x 2^e, so none underflows), and sig = 2^f with
// sig ||x|| < 2^13 (the scale of the second product's operand when the
// rotated row itself is handed on, as in query preparation).  Zero rows get
// nx = 0 and unit scales.
__global__ __launch_bounds__(256) void rowscale_kernel(const void* x, int bf16, int64_t ld, int64_t rows, int d,
                                                       float* sc, float* nx, float* sig) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  // fp32 rows are read once, 16 bytes per lane per step, and kept in
  // registers (d <= 4096: at most 16 steps of 256 elements); bf16 rows take a
  // strided two-pass form
  constexpr int MAXS = 16;
  float4 v[MAXS];
#pragma unroll
  for (int u = 0; u < MAXS; ++u) {
    v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int i0 = u * 256 + lane * 4;
    if (!bf16 && i0 < d) v[u] = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + row * ld + i0);
  }
  float mx = 0.f;
  if (bf16) {
    for (int i = lane; i < d; i += 64)
      mx = fmaxf(mx, fabsf(__uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[row * ld + i]) << 16)));
  } else {
#pragma unroll
    for (int u = 0; u < MAXS; ++u)
      mx = fmaxf(fmaxf(fmaxf(mx, fabsf(v[u].x)), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const int eb = int((__float_as_uint(mx) >> 23) & 0xff);
  const float p2 = mx > 0.f ? __uint_as_float(uint32_t(min(253, max(1, 268 - eb))) << 23) : 1.f;
  // the squares are summed over x 2^e, so none underflows
  float ss = 0.f;
  if (bf16) {
    for (int i = lane; i < d; i += 64) {
      const float t = __uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[row * ld + i]) << 16) * p2;
      ss = fmaf(t, t, ss);
    }
  } else {
#pragma unroll
    for (int u = 0; u < MAXS; ++u) {
      const float a0 = v[u].x * p2, a1 = v[u].y * p2, a2 = v[u].z * p2, a3 = v[u].w * p2;
      ss = fmaf(a0, a0, fmaf(a1, a1, fmaf(a2, a2, fmaf(a3, a3, ss))));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) {
    const float n = sqrtf(ss) / p2;
    sc[row] = p2;
    nx[row] = n;
    const int en = int((__float_as_uint(n) >> 23) & 0xff);  // n in [2^(en-127), 2^(en-126))
    sig[row] = n > 0.f ? __uint_as_float(uint32_t(min(253, max(1, 127 + 139 - en))) << 23) : 1.f;
  }
}

// ------------------------------------------------------------- rotate
struct RotArgs {
  const void* x;            // chunk rows, fp32 or bf16, row stride ld elements
  int64_t ld;
  int64_t rows_valid;       // rows of x in the chunk
  int64_t rows_out;         // rows that own a record slot (>= rows_valid)
  int d;
  const float* sc;          // [rows] input scale 2^e
  const float* nx;          // [rows] norms
  const float* sig;         // [rows] scale of the handed-on rotated row (query preparation)
  const uint16_t* tiles;    // Pi tiles: [d/128][d/32][hi, lo][128][32], rows in lds_row order
  // encode
  uint8_t* rec;             // records of the chunk's first row (a tile boundary)
  int tile_bytes, off_nx;
  float thr[kMaxLevels - 1], cen[kMaxLevels];
  uint16_t* rhi;            // [rows][d] fp16 parts of 2^13 r (prod), or of sig y (query preparation)
  uint16_t* rlo;
  float* rr;                // [rows][d/128] partial sums of (2^13 r)^2 (prod)
  // query preparation
  float* yout;              // [rows][d] y = Pi x
};

// Coordinate of accumulator register r of lane half h in 32-row block c:
// the tiles hold the rows of each 32-row group permuted so that a half-wave
// owns 16 consecutive coordinates, 32 c + 16 h + r.
template <bool XBF16, int MODE, int UB>  // MODE 0: encode mse, 1: encode prod, 2: query preparation
__global__ __launch_bounds__(NT, 2) void rotate_kernel(RotArgs a) {
  __shared__ __align__(16) uint16_t sA[2][2 * AR * AP];
  __shared__ float scen[kMaxLevels];
  const int ncb = a.d / 128, nkt = a.d / KT;
  const int nrt = int((a.rows_out + BW - 1) / BW);
  int rt, cb;
  if (!map_tile(nrt, ncb, rt, cb)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 31, h = lane >> 5;
  if (threadIdx.x < kMaxLevels) scen[threadIdx.x] = a.cen[threadIdx.x] * kRScale;

  int64_t row[2];
  bool valid[2];
  const uint8_t* xp[2];
  float scv[2];
  const int esz = XBF16 ? 2 : 4;
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    row[v] = int64_t(rt) * BW + 64 * wave + 32 * v + j;
    valid[v] = row[v] < a.rows_valid;
    const int64_t lr = valid[v] ? row[v] : a.rows_valid - 1;
    xp[v] = static_cast<const uint8_t*>(a.x) + (lr * a.ld + 16 * h) * esz;
    scv[v] = a.sc[lr];
  }
  // raw B rows of one tile: 16 elements per row (64 bytes fp32, 32 bytes bf16)
  constexpr int NR = XBF16 ? 2 : 4;
  u32x4 raw[2][NR], nraw[2][NR];
  auto load_b = [&](int kt, u32x4 (&dst)[2][NR]) {
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int u = 0; u < NR; ++u) dst[v][u] = reinterpret_cast<const u32x4*>(xp[v] + int64_t(kt) * KT * esz)[u];
  };
  const uint16_t* tile0 = a.tiles + size_t(cb) * nkt * (2 * AR * KT);
  // the tile's B operands: x 2^e as fp16 hi (+ lo for fp32 input)
  u32x4 bh[2][2], bl[2][2];
  auto convert = [&](const u32x4 (&src)[2][NR]) {
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float f[8];
        if (XBF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = src[v][s][e];
            f[2 * e] = __uint_as_float(w << 16) * scv[v];
            f[2 * e + 1] = __uint_as_float(w & 0xffff0000u) * scv[v];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) bh[v][s][e] = h16(f[2 * e]) | (h16(f[2 * e + 1]) << 16);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = __uint_as_float(src[v][2 * s + e / 4][e % 4]) * scv[v];
          split8(f, bh[v][s], bl[v][s]);
        }
      }
  };
  AStage<2> st;
  st.load(tile0);
  load_b(0, raw);
  st.store(sA[0]);
  convert(raw);
  __syncthreads();

  f32x16 acc[4][2];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 2; ++v) acc[c][v] = f32x16{};

  for (int kt = 0; kt < nkt; ++kt) {
    // the next tile's loads first (clamped to the last tile: unconditional,
    // so the wait counters stay exact across the loop)
    const int kn = min(kt + 1, nkt - 1);
    st.load(tile0 + size_t(kn) * (2 * AR * KT));
    load_b(kn, nraw);
    const uint16_t* L = sA[kt & 1];
    // 8 steps (s, c): the Pi fragments of step i + 1 are read from LDS while
    // the 6 MFMAs of step i run
    u32x4 ah[2], al[2];
    ah[0] = afrag(L, 0, 0, 0, lane);
    al[0] = afrag(L, 1, 0, 0, lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = i >> 2, c = i & 3;
      if (i + 1 < 8) {
        ah[(i + 1) & 1] = afrag(L, 0, (i + 1) & 3, (i + 1) >> 2, lane);
        al[(i + 1) & 1] = afrag(L, 1, (i + 1) & 3, (i + 1) >> 2, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        acc[c][v] = mfma(ah[i & 1], bh[v][s], acc[c][v]);
        acc[c][v] = mfma(al[i & 1], bh[v][s], acc[c][v]);
        if (!XBF16) acc[c][v] = mfma(ah[i & 1], bl[v][s], acc[c][v]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    convert(nraw);
    st.store(sA[(kt + 1) & 1]);
    __syncthreads();
  }

  // ---- epilogue: acc[c][v][r] = 16 2^e (Pi x) of coordinate 128 cb + 32 c + 16 h + r
  const int coord0 = 128 * cb + 16 * h;
  if (MODE == 2) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      if (!valid[v]) continue;
      const float back = 1.f / (16.f * scv[v]);
      const float sg = a.sig[row[v]] * back;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float y[16], ys[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          y[r] = acc[c][v][r] * back;
          ys[r] = acc[c][v][r] * sg;
        }
        float* yo = a.yout + row[v] * a.d + coord0 + 32 * c;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          reinterpret_cast<float4*>(yo)[q] = make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
        u32x4 hi[2], lo[2];
        split8(*reinterpret_cast<const float(*)[8]>(&ys[0]), hi[0], lo[0]);
        split8(*reinterpret_cast<const float(*)[8]>(&ys[8]), hi[1], lo[1]);
        uint16_t* ph = a.rhi + row[v] * a.d + coord0 + 32 * c;
        uint16_t* pl = a.rlo + row[v] * a.d + coord0 + 32 * c;
        reinterpret_cast<u32x4*>(ph)[0] = hi[0];
        reinterpret_cast<u32x4*>(ph)[1] = hi[1];
        reinterpret_cast<u32x4*>(pl)[0] = lo[0];
        reinterpret_cast<u32x4*>(pl)[1] = lo[1];
      }
    }
    return;
  }
  constexpr int NTH = (1 << UB) - 1;
  float T[2][NTH], inv[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const float n = a.nx[valid[v] ? row[v] : a.rows_valid - 1];
    const float w = 16.f * scv[v] * (n > 0.f ? n : 1.f);  // a zero row encodes y = 0
#pragma unroll
    for (int t = 0; t < NTH; ++t) T[v][t] = a.thr[t] * w;
    inv[v] = kRScale / w;
  }
  uint32_t planes[UB][4][2];  // [plane][c][v]: 16 bits of this half's coordinates
  float rsum[2] = {0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
#pragma unroll
      for (int p = 0; p < UB; ++p) planes[p][c][v] = 0u;
      float rs[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float y = acc[c][v][r];
        int idx = 0;
#pragma unroll
        for (int t = 0; t < NTH; ++t) idx += y >= T[v][t] ? 1 : 0;
#pragma unroll
        for (int p = 0; p < UB; ++p) planes[p][c][v] |= uint32_t((idx >> p) & 1) << r;
        if (MODE == 1) {
          rs[r] = fmaf(y, inv[v], -scen[idx]);
          rsum[v] = fmaf(rs[r], rs[r], rsum[v]);
        }
      }
      if (MODE == 1 && valid[v]) {
        u32x4 hi[2], lo[2];
        split8(*reinterpret_cast<const float(*)[8]>(&rs[0]), hi[0], lo[0]);
        split8(*reinterpret_cast<const float(*)[8]>(&rs[8]), hi[1], lo[1]);
        uint16_t* ph = a.rhi + row[v] * a.d + coord0 + 32 * c;
        uint16_t* pl = a.rlo + row[v] * a.d + coord0 + 32 * c;
        reinterpret_cast<u32x4*>(ph)[0] = hi[0];
        reinterpret_cast<u32x4*>(ph)[1] = hi[1];
        reinterpret_cast<u32x4*>(pl)[0] = lo[0];
        reinterpret_cast<u32x4*>(pl)[1] = lo[1];
      }
      // one block at a time: keeps the scheduler from hoisting every block's
      // table reads (and their registers) to the top
      __builtin_amdgcn_sched_barrier(0);
    }
  // lane half h stores the records of vector block v = h: exchange halves
  const int64_t orow = int64_t(rt) * BW + 64 * wave + 32 * h + j;  // this lane's output vector
  const bool ovalid = orow < a.rows_valid, oslot = orow < a.rows_out;
  uint8_t* trec = a.rec + (orow / kTile) * a.tile_bytes;
  const int slot = int(orow % kTile);
#pragma unroll
  for (int p = 0; p < UB; ++p) {
    u32x4 wv;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t t = planes[p][c][0] | (planes[p][c][1] << 16);
      const uint32_t u = uint32_t(__shfl_xor(int(t), 32, 64));
      wv[c] = h == 0 ? ((t & 0xffffu) | (u << 16)) : ((u >> 16) | (t & 0xffff0000u));
    }
    if (!ovalid) wv = u32x4{0u, 0u, 0u, 0u};
    if (oslot)
      *reinterpret_cast<u32x4*>(trec + size_t(p * ncb + cb) * kTile * 16 + size_t(slot) * 16) = wv;
  }
  if (MODE == 1) {
    const float r0 = rsum[0] + __shfl_xor(rsum[0], 32, 64);
    const float r1 = rsum[1] + __shfl_xor(rsum[1], 32, 64);
    if (ovalid) a.rr[orow * ncb + cb] = h == 0 ? r0 : r1;
  }
  if (cb == 0 && oslot) {
    const float n = ovalid ? a.nx[orow] : 0.f;
    *reinterpret_cast<uint16_t*>(trec + a.off_nx + 2 * slot) = uint16_t(h16(n));
  }
}

// ------------------------------------------------------------- sketch
struct SketchArgs {
  const uint16_t* rhi;      // [rows][m] fp16 parts of the scaled rows
  const uint16_t* rlo;
  int64_t rows_valid, rows_out;
  int m;
  const uint16_t* tiles;    // S tiles: [m/128][m/32][128][32], rows in lds_row order
  // encode: signs and n_r
  uint8_t* rec;
  int tile_bytes, off_signs, off_nr;
  const float* rr;          // [rows][m/128]
  // query preparation: qs = z / sig
  const float* sig;
  float* zout;              // [rows][m]
};

template <int MODE>  // 0: encode (signs, n_r), 1: query preparation
__global__ __launch_bounds__(NT, 2) void sketch_kernel(SketchArgs a) {
  __shared__ __align__(16) uint16_t sA[2][AR * AP];
  const int ncb = a.m / 128, nkt = a.m / KT;
  const int nrt = int((a.rows_out + BW - 1) / BW);
  int rt, cb;
  if (!map_tile(nrt, ncb, rt, cb)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 31, h = lane >> 5;
  int64_t row[2];
  bool valid[2];
  const uint16_t *ph[2], *pl[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    row[v] = int64_t(rt) * BW + 64 * wave + 32 * v + j;
    valid[v] = row[v] < a.rows_valid;
    const int64_t lr = valid[v] ? row[v] : a.rows_valid - 1;
    ph[v] = a.rhi + lr * a.m + 16 * h;
    pl[v] = a.rlo + lr * a.m + 16 * h;
  }
  u32x4 bh[2][2], bl[2][2], nbh[2][2], nbl[2][2];
  auto load_b = [&](int kt, u32x4 (&dh)[2][2], u32x4 (&dl)[2][2]) {
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        dh[v][s] = reinterpret_cast<const u32x4*>(ph[v] + kt * KT)[s];
        dl[v][s] = reinterpret_cast<const u32x4*>(pl[v] + kt * KT)[s];
      }
  };
  const uint16_t* tile0 = a.tiles + size_t(cb) * nkt * (AR * KT);
  AStage<1> st;
  st.load(tile0);
  load_b(0, bh, bl);
  st.store(sA[0]);
  __syncthreads();
  f32x16 acc[4][2];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 2; ++v) acc[c][v] = f32x16{};
  for (int kt = 0; kt < nkt; ++kt) {
    // the next tile's loads first (clamped, unconditional: exact wait counters)
    const int kn = min(kt + 1, nkt - 1);
    st.load(tile0 + size_t(kn) * (AR * KT));
    load_b(kn, nbh, nbl);
    const uint16_t* L = sA[kt & 1];
    // 8 steps (s, c): the S fragment of step i + 1 is read while the 4
    // MFMAs of step i run
    u32x4 af[2];
    af[0] = afrag(L, 0, 0, 0, lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = i >> 2, c = i & 3;
      if (i + 1 < 8) af[(i + 1) & 1] = afrag(L, 0, (i + 1) & 3, (i + 1) >> 2, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        acc[c][v] = mfma(af[i & 1], bh[v][s], acc[c][v]);
        acc[c][v] = mfma(af[i & 1], bl[v][s], acc[c][v]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    st.store(sA[(kt + 1) & 1]);
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bh[v][s] = nbh[v][s];
        bl[v][s] = nbl[v][s];
      }
    __syncthreads();
  }
  const int coord0 = 128 * cb + 16 * h;
  if (MODE == 1) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      if (!valid[v]) continue;
      const float back = 1.f / a.sig[row[v]];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float* zo = a.zout + row[v] * a.m + coord0 + 32 * c;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          reinterpret_cast<float4*>(zo)[q] = make_float4(acc[c][v][4 * q] * back, acc[c][v][4 * q + 1] * back,
                                                         acc[c][v][4 * q + 2] * back, acc[c][v][4 * q + 3] * back);
      }
    }
    return;
  }
  // sign bits [z >= 0] (an accumulator is never -0)
  const int64_t orow = int64_t(rt) * BW + 64 * wave + 32 * h + j;
  const bool ovalid = orow < a.rows_valid, oslot = orow < a.rows_out;
  uint8_t* trec = a.rec + (orow / kTile) * a.tile_bytes;
  const int slot = int(orow % kTile);
  u32x4 wv;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t b2[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      uint32_t b = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) b |= uint32_t(acc[c][v][r] >= 0.f) << r;
      b2[v] = b;
    }
    const uint32_t t = b2[0] | (b2[1] << 16);
    const uint32_t u = uint32_t(__shfl_xor(int(t), 32, 64));
    wv[c] = h == 0 ? ((t & 0xffffu) | (u << 16)) : ((u >> 16) | (t & 0xffff0000u));
  }
  if (!ovalid) wv = u32x4{0u, 0u, 0u, 0u};
  if (oslot) *reinterpret_cast<u32x4*>(trec + a.off_signs + size_t(cb) * kTile * 16 + size_t(slot) * 16) = wv;
  if (cb == 0 && oslot) {
    float ss = 0.f;
    if (ovalid)
      for (int b = 0; b < ncb; ++b) ss += a.rr[orow * ncb + b];
    const float nr = ovalid ? sqrtf(ss) / kRScale : 0.f;
    *reinterpret_cast<uint16_t*>(trec + a.off_nr + 2 * slot) = uint16_t(h16(nr));
  }
}

// ------------------------------------------------------------- query tiles
// One wave per query row of the search operand: the row
// [kqjl qs | fc q'] (prod; [fc q'] for mse), scaled by 2^e so that its
// largest entry lies in [2^14, 2^15), in fp16, written to the query tiles
// [nq/128][K/128][128 rows][128 elements]; inv[q] = 2^-e.  Rows past nq are
// zero.
constexpr int SK = 128;  // reduction elements per search tile: one record chunk
__global__ __launch_bounds__(256) void qtiles_kernel(const float* qr, const float* qs, int64_t nq, int64_t nrows,
                                                     int d, int m, float kq, float fc, uint16_t* tiles,
                                                     float* inv) {
  const int lane = threadIdx.x & 63;
  const int64_t q = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (q >= nrows) return;
  const int K = d + m, nkt = K / SK;
  const bool real = q < nq;
  auto at = [&](int i) -> float {
    if (!real) return 0.f;
    return i < m ? kq * qs[q * m + i] : fc * qr[q * d + (i - m)];
  };
  float mx = 0.f;
  for (int i = lane; i < K; i += 64) mx = fmaxf(mx, fabsf(at(i)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const int eb = int((__float_as_uint(mx) >> 23) & 0xff);
  const int e = mx > 0.f ? min(253, max(1, 268 - eb)) : 127;
  const float p2 = __uint_as_float(uint32_t(e) << 23);
  uint16_t* base = tiles + (q / AR) * int64_t(nkt) * AR * SK + (q % AR) * SK;
  for (int i = lane; i < K; i += 64) base[int64_t(i / SK) * AR * SK + (i % SK)] = uint16_t(h16(at(i) * p2));
  if (lane == 0) inv[q] = real && mx > 0.f ? __uint_as_float(uint32_t(254 - e) << 23) : 0.f;
}

// ------------------------------------------------------------- search
struct SearchArgs {
  const uint16_t* qtiles;   // [nqb][K/32][128][32]
  const float* inv;         // [nqb * 128] query scales (0 for padding rows)
  int64_t nq;
  int nqb;
  const uint8_t* rec;
  int64_t n;
  int d, m;                 // m = 0 for mse codecs
  int tile_bytes, off_signs, off_nx, off_nr;
  float cen[8];             // levels of the 2- and 3-bit codebooks
  int nsplit;
  int64_t keys_per_split;   // a multiple of the workgroup's keys per tile
  int k;                    // list length (top-k)
  int nparts;               // partial lists per query = 4 * nsplit
  float* ps;                // [nq][nparts][k]
  int64_t* pi;
  int* thr;                 // [nqb * 128] shared admission thresholds (order-preserving int of a float)
  float* scores;            // dense output [nq][n]
};

// Order-preserving map of floats (not NaN) to ints, so that thresholds can be
// raised with an integer atomic max.
__device__ __forceinline__ int ord_of(float f) {
  const int i = __float_as_int(f);
  return i >= 0 ? i : i ^ 0x7fffffff;
}
__device__ __forceinline__ float float_of_ord(int i) { return __int_as_float(i >= 0 ? i : i ^ 0x7fffffff); }

__global__ void fill_ord_kernel(int* p, int64_t n, float v) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = ord_of(v);
}

__device__ __forceinline__ bool better(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

template <int KM>
struct TopList {
  float s[KM];
  int id[KM];
  float ts;   // entry k - 1, the admission threshold
  int ti;
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < KM; ++t) { s[t] = -INFINITY; id[t] = 0x7fffffff; }
    ts = -INFINITY;
    ti = 0x7fffffff;
  }
  // insert (cs, ci), known to beat entry k - 1
  __device__ __forceinline__ void insert(float cs, int ci, int k) {
    float ns[KM];
    int ni[KM];
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      const bool here = better(cs, ci, s[t], id[t]);
      const bool above = t > 0 && better(cs, ci, s[t > 0 ? t - 1 : 0], id[t > 0 ? t - 1 : 0]);
      ns[t] = above ? s[t > 0 ? t - 1 : 0] : (here ? cs : s[t]);
      ni[t] = above ? id[t > 0 ? t - 1 : 0] : (here ? ci : id[t]);
    }
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      s[t] = ns[t];
      id[t] = ni[t];
      if (t == k - 1) { ts = ns[t]; ti = ni[t]; }
    }
  }
};

// Key operand tables: byte -> 8 fp16 of +-1 (bit set: +1), and for 2 or 3
// index bits per coordinate, 4 coordinates' plane nibbles -> their 4 fp16
// centroids (index n0 | n1 << 4 | n2 << 8, coordinate e's index from bit e of
// each nibble).
template <int UB>
struct KeyTables {
  static constexpr int NC = UB == 2 ? 256 : (UB == 3 ? 4096 : 1);
  u32x4 pm[256];
  u32x2 cen[NC];
};

// NV: 32-key blocks per wave (the workgroup takes 128 NV keys at a time).
// QW: waves per key block.  QW = 1: 4 waves, each computing all 128 queries
// of the block for its keys (one wave per SIMD: 4 x NV accumulator blocks and
// two top-k lists per lane); QW = 2: 8 waves, wave w computing queries
// 64 (w / 4) .. + 63 for the keys of sub-block w % 4, so that two waves share
// each SIMD (2 x NV accumulator blocks, one list per lane) at the price of
// reading each key operand twice.
template <int UB, bool PROD, bool DENSE, int KM, int NV, int QW>  // KM: list slots (k <= KM)
__global__ __launch_bounds__(NT * QW, 1) void search_kernel(SearchArgs a) {
  constexpr int NTS = NT * QW;  // threads
  constexpr int CQ = 4 / QW;    // 32-query row blocks per wave
  constexpr int NL = CQ / 2;    // top-k lists per lane (64 queries each)
  constexpr int TP = 33;        // pitch of the transposition buffer (floats)
  constexpr int SP = SK + 8;    // LDS pitch of a query row (halves): 272 bytes, conflict-free 16-byte reads
  __shared__ __align__(16) uint16_t sA[2][AR * SP];
  __shared__ __align__(16) KeyTables<UB> tb;
  __shared__ float sinv[AR];
  __shared__ float sT[DENSE ? 1 : 4 * QW][DENSE ? 1 : 64 * TP];
  const int qb = blockIdx.x % a.nqb, split = blockIdx.x / a.nqb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 31, h = lane >> 5;
  const int kw = wave & 3;                        // key sub-block of the wave
  const int qbase = QW == 2 ? 64 * (wave >> 2) : 0;  // first query row of the wave
  const int tid = threadIdx.x;
  // tables
  {
    if (tid < 256) {
      const uint32_t b = uint32_t(tid);
      u32x4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        e[i] = ((b >> (2 * i)) & 1u ? 0x3c00u : 0xbc00u) | (((b >> (2 * i + 1)) & 1u ? 0x3c00u : 0xbc00u) << 16);
      tb.pm[b] = e;
    }
    if (UB >= 2) {
      for (int t = tid; t < KeyTables<UB>::NC; t += NTS) {
        uint32_t hv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          int idx = int((t >> c) & 1) | (int((t >> (4 + c)) & 1) << 1);
          if (UB == 3) idx |= int((t >> (8 + c)) & 1) << 2;
          hv[c] = h16(a.cen[idx]);
        }
        tb.cen[t] = u32x2{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
      }
    }
    if (tid < AR) sinv[tid] = a.inv[int64_t(qb) * AR + tid];
  }
  const int m = PROD ? a.m : 0;
  const int GS = m / SK, GC = a.d / SK;  // tiles (= record chunks): signs, then codes
  const int nkt = GS + GC;
  const uint16_t* qt = a.qtiles + size_t(qb) * nkt * (AR * SK);
  const int64_t k0 = int64_t(split) * a.keys_per_split;
  const int64_t k1 = min(a.n, k0 + a.keys_per_split);
  // list hl of a lane holds query 128 qb + qbase + 64 hl + lane
  TopList<KM> Ls[NL];
  float invs[NL];
#pragma unroll
  for (int hl = 0; hl < NL; ++hl) {
    Ls[hl].init();
    invs[hl] = DENSE ? 0.f : a.inv[int64_t(qb) * AR + qbase + 64 * hl + lane];
  }
  __syncthreads();

  // query tile staging: 32 KB per tile, 16 bytes per chunk, NS chunks per thread
  constexpr int NS = AR * SK / 8 / NTS;
  u32x4 stg[NS];
  auto stage_load = [&](int kt) {
    const u32x4* g = reinterpret_cast<const u32x4*>(qt + size_t(kt) * (AR * SK));
#pragma unroll
    for (int u = 0; u < NS; ++u) stg[u] = g[u * NTS + tid];
  };
  auto stage_store = [&](uint16_t* lds) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int e = u * NTS + tid, row = e / (SK / 8), c8 = e % (SK / 8);
      *reinterpret_cast<u32x4*>(lds + row * SP + c8 * 8) = stg[u];
    }
  };

  constexpr int WK = 32 * NV;  // keys per wave
  for (int64_t kb = k0; kb < k1; kb += 4 * WK) {
    int64_t key[NV];
    bool kval[NV];
    const uint8_t* kt0[NV];
    int kslot[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      key[v] = kb + WK * kw + 32 * v + j;
      kval[v] = key[v] < k1;
      const int64_t lk = kval[v] ? key[v] : k1 - 1;
      kt0[v] = a.rec + (lk / kTile) * a.tile_bytes;
      kslot[v] = int(lk % kTile);
    }
    // record chunks of tile kt: the sign chunk kt (kt < GS), else chunk kt - GS
    // of every code plane (branch-free: the sign tiles read the sign chunk
    // into every plane register)
    auto load_chunks = [&](int kt, u32x4 (&dst)[NV][UB]) {
      const bool sg = PROD && kt < GS;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int p = 0; p < UB; ++p) {
          const size_t off = sg ? size_t(a.off_signs) + size_t(kt) * kTile * 16
                                : size_t(p * GC + kt - GS) * kTile * 16;
          dst[v][p] = *reinterpret_cast<const u32x4*>(kt0[v] + off + size_t(kslot[v]) * 16);
        }
    };
    u32x4 cw[NV][UB], ncw[NV][UB];
    stage_load(0);
    load_chunks(0, cw);
    stage_store(sA[0]);
    __syncthreads();
    f32x16 acc[CQ][NV];
#pragma unroll
    for (int c = 0; c < CQ; ++c)
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[c][v] = f32x16{};
    // One tile of 128 reduction elements; the next tile's query rows and
    // record chunks are loaded first (clamped to the last tile: the loads are
    // unconditional, so the wait counters stay exact across the loop).
    auto tile = [&](int kt, auto signs_c) {
      constexpr bool SIGNS = decltype(signs_c)::value;
      const int kn = min(kt + 1, nkt - 1);
      stage_load(kn);
      load_chunks(kn, ncw);
      const uint16_t* LA = sA[kt & 1];
      // 8 MFMA steps of 16: step t = (kq, s) takes elements 32 kq + 16 h + 8 s .. + 7.
      // The LDS reads of step t + 1 (query fragments, key table rows) are
      // issued before the MFMAs of step t, so their latency hides behind them.
      auto read_step = [&](int t, u32x4 (&af)[CQ], u32x4 (&bf)[NV]) {
        const int kq = t >> 1, s = t & 1;
        const int sh = 16 * h + 8 * s;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          if (SIGNS || UB == 1) {
            bf[v] = tb.pm[(cw[v][0][kq] >> sh) & 0xffu];
          } else {
            const uint32_t b0 = (cw[v][0][kq] >> sh) & 0xffu, b1 = (cw[v][UB > 1 ? 1 : 0][kq] >> sh) & 0xffu;
            uint32_t ilo = (b0 & 15u) | ((b1 & 15u) << 4), ihi = (b0 >> 4) | (b1 & 0xf0u);
            if (UB == 3) {
              const uint32_t b2 = (cw[v][UB == 3 ? 2 : 0][kq] >> sh) & 0xffu;
              ilo |= (b2 & 15u) << 8;
              ihi |= (b2 & 0xf0u) << 4;
            }
            const u32x2 lo = tb.cen[ilo], hi = tb.cen[ihi];
            bf[v] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
        }
#pragma unroll
        for (int c = 0; c < CQ; ++c)
          af[c] = *reinterpret_cast<const u32x4*>(LA + (qbase + 32 * c + j) * SP + 32 * kq + 16 * h + 8 * s);
      };
      auto mma_step = [&](const u32x4 (&af)[CQ], const u32x4 (&bf)[NV]) {
#pragma unroll
        for (int c = 0; c < CQ; ++c)
#pragma unroll
          for (int v = 0; v < NV; ++v) acc[c][v] = mfma(af[c], bf[v], acc[c][v]);
      };
      // The reads of step t + 1 are interleaved with the 8 MFMAs of step t
      // (one MFMA, then an LDS read and a few ALU instructions, eight times),
      // so that they issue while the matrix core is busy.
      auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < CQ * NV; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // up to three VALU
        }
      };
      u32x4 afA[CQ], bfA[NV], afB[CQ], bfB[NV];
      read_step(0, afA, bfA);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        read_step(t + 1, afB, bfB);
        mma_step(afA, bfA);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        if (t + 2 < 8) read_step(t + 2, afA, bfA);
        mma_step(afB, bfB);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
      }
      stage_store(sA[(kt + 1) & 1]);
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int p = 0; p < UB; ++p) cw[v][p] = ncw[v][p];
      __syncthreads();
    };
    for (int kt = 0; kt < GS; ++kt) tile(kt, std::integral_constant<bool, true>{});
    if (PROD) {
      // between the sign phase and the code phase: acc *= n_r of the key
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const float nr = f16f(*reinterpret_cast<const uint16_t*>(kt0[v] + a.off_nr + 2 * kslot[v]));
#pragma unroll
        for (int c = 0; c < CQ; ++c) acc[c][v] *= nr;
      }
    }
    for (int kt = GS; kt < nkt; ++kt) tile(kt, std::integral_constant<bool, false>{});
    // ---- epilogue: s = acc n_x inv_q; acc[c][v][r] is query qbase + 32 c + 8 (r / 4) + 4 h + r % 4, key v
    float nxv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
      nxv[v] = kval[v] ? f16f(*reinterpret_cast<const uint16_t*>(kt0[v] + a.off_nx + 2 * kslot[v])) : 0.f;
    if (DENSE) {
#pragma unroll
      for (int c = 0; c < CQ; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = qbase + 32 * c + 8 * (r >> 2) + 4 * h + (r & 3);
          const int64_t q = int64_t(qb) * AR + qrow;
          if (q >= a.nq) continue;
          const float iq = sinv[qrow];
#pragma unroll
          for (int v = 0; v < NV; ++v)
            if (kval[v]) a.scores[q * a.n + key[v]] = acc[c][v][r] * nxv[v] * iq;
        }
      continue;
    }
    float* T = sT[wave];
    // A key can enter the final top-k of a query only if its score reaches
    // the shared threshold: the k-th best score of some partial list, which
    // never exceeds the final k-th best.  Every list raises the shared value
    // (an integer atomic max) after each workgroup tile, so all workgroups of
    // the query block filter against it.
#pragma unroll
    for (int hq = 0; hq < NL; ++hq) {
      TopList<KM>& Lq = Ls[hq];
      const float iq = invs[hq];
      int* tq = a.thr + int64_t(qb) * AR + qbase + 64 * hq + lane;
      const float tg = float_of_ord(__hip_atomic_load(tq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      const float ts0 = Lq.ts;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        // queries 64 hq .. 64 hq + 63 x keys 32 v .. 32 v + 31 of the wave, via LDS
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            T[(32 * c2 + 8 * (r >> 2) + 4 * h + (r & 3)) * TP + j] = acc[2 * hq + c2][v][r] * nxv[v];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int kbase = int(kb) + WK * kw + 32 * v;  // key id of column 0 (n < 2^31)
        const int kvalid = int(min<int64_t>(32, max<int64_t>(0, k1 - (kb + WK * kw + 32 * v))));
        const float* row = T + lane * TP;
        uint32_t cand = 0;
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) {
          const float sc = row[jj] * iq;
          if (jj < kvalid && sc >= tg && better(sc, kbase + jj, Lq.ts, Lq.ti)) cand |= 1u << jj;
        }
        while (cand) {
          const int jj = __builtin_ctz(cand);
          cand &= cand - 1;
          const float cs = row[jj] * iq;
          if (better(cs, kbase + jj, Lq.ts, Lq.ti)) Lq.insert(cs, kbase + jj, a.k);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      if (Lq.ts > ts0 && Lq.ts > tg) atomicMax(tq, ord_of(Lq.ts));
    }
  }
  if (DENSE) return;
  // partial lists of this wave: part (split, key sub-block) of each query
  const int part = split * 4 + kw;
#pragma unroll
  for (int hq = 0; hq < NL; ++hq) {
    const int64_t q = int64_t(qb) * AR + qbase + 64 * hq + lane;
    if (q >= a.nq) continue;
    const TopList<KM>& Lq = Ls[hq];
    float* ps = a.ps + (q * a.nparts + part) * a.k;
    int64_t* pi = a.pi + (q * a.nparts + part) * a.k;
#pragma unroll
    for (int t = 0; t < KM; ++t)
      if (t < a.k) {
        ps[t] = Lq.s[t];
        pi[t] = Lq.id[t] == 0x7fffffff ? int64_t(INT64_MAX) : int64_t(Lq.id[t]);
      }
  }
}

unsigned blocks_of(int64_t threads, int bs = 256) { return unsigned((threads + bs - 1) / bs); }

}  // namespace

// ------------------------------------------------------------------ host side
int64_t wide_encode_chunk() { return 32768; }

namespace {
struct EncodeWs {
  float *sc, *nx, *sig, *rr;
  uint16_t *rhi, *rlo;
};
size_t encode_ws(const CodecView& cv, int64_t rows, void* base, EncodeWs* o) {
  const size_t R = size_t(rows), d = size_t(cv.d);
  auto rnd = [](size_t v) { return (v + 255) & ~size_t(255); };
  const bool prod = cv.mode == TQ_PROD;
  const size_t sizes[6] = {rnd(R * 4), rnd(R * 4), rnd(R * 4), prod ? rnd(R * (d / 128) * 4) : 0,
                           prod ? rnd(R * d * 2) : 0, prod ? rnd(R * d * 2) : 0};
  size_t off[6], tot = 0;
  for (int i = 0; i < 6; ++i) { off[i] = tot; tot += sizes[i]; }
  if (o) {
    uint8_t* p = static_cast<uint8_t*>(base);
    o->sc = reinterpret_cast<float*>(p + off[0]);
    o->nx = reinterpret_cast<float*>(p + off[1]);
    o->sig = reinterpret_cast<float*>(p + off[2]);
    o->rr = reinterpret_cast<float*>(p + off[3]);
    o->rhi = reinterpret_cast<uint16_t*>(p + off[4]);
    o->rlo = reinterpret_cast<uint16_t*>(p + off[5]);
  }
  return tot;
}

hipError_t launch_rotate(const CodecView& cv, int mode, bool bf16, const RotArgs& ra, hipStream_t s) {
  const int nrt = int((ra.rows_out + BW - 1) / BW);
  const dim3 grid(unsigned((nrt + 7) / 8 * 8 * (cv.d / 128)));
#define TQ_ROT(XB, MD, U) hipLaunchKernelGGL((rotate_kernel<XB, MD, U>), grid, dim3(NT), 0, s, ra)
#define TQ_ROT_UB(XB, MD)                         \
  switch (cv.ubits) {                             \
    case 1: TQ_ROT(XB, MD, 1); break;             \
    case 2: TQ_ROT(XB, MD, 2); break;             \
    case 3: TQ_ROT(XB, MD, 3); break;             \
    case 4: TQ_ROT(XB, MD, 4); break;             \
    case 5: TQ_ROT(XB, MD, 5); break;             \
    default: return hipErrorNotSupported;         \
  }
  if (mode == 2) {
    if (bf16) TQ_ROT(true, 2, 1); else TQ_ROT(false, 2, 1);
  } else if (mode == 1) {
    if (bf16) { TQ_ROT_UB(true, 1) } else { TQ_ROT_UB(false, 1) }
  } else {
    if (bf16) { TQ_ROT_UB(true, 0) } else { TQ_ROT_UB(false, 0) }
  }
#undef TQ_ROT_UB
#undef TQ_ROT
  return hipGetLastError();
}

hipError_t launch_sketch(const CodecView& cv, int mode, const SketchArgs& sa, hipStream_t s) {
  const int nrt = int((sa.rows_out + BW - 1) / BW);
  const dim3 grid(unsigned((nrt + 7) / 8 * 8 * (cv.m / 128)));
  if (mode == 1)
    hipLaunchKernelGGL((sketch_kernel<1>), grid, dim3(NT), 0, s, sa);
  else
    hipLaunchKernelGGL((sketch_kernel<0>), grid, dim3(NT), 0, s, sa);
  return hipGetLastError();
}
}  // namespace

size_t wide_encode_workspace(const CodecView& cv) { return encode_ws(cv, wide_encode_chunk(), nullptr, nullptr); }

hipError_t launch_encode_wide(const CodecView& cv, const EncodeArgs& a, void* ws, hipStream_t s) {
  const int64_t C = wide_encode_chunk();
  const bool prod = cv.mode == TQ_PROD;
  EncodeWs W;
  encode_ws(cv, C, ws, &W);
  const int esz = a.x_bf16 ? 2 : 4;
  const int64_t padded = (a.tokens + kTile - 1) / kTile * kTile;
  hipError_t e;
  for (int64_t b = 0; b < a.batch; ++b)
    for (int64_t hh = 0; hh < a.heads; ++hh) {
      const uint8_t* xs = static_cast<const uint8_t*>(a.x) + (b * a.xs_b + hh * a.xs_h) * esz;
      uint8_t* rec = a.rec + b * a.rs_b + hh * a.rs_h;
      for (int64_t r0 = 0; r0 < padded; r0 += C) {
        const int64_t rows_out = std::min(C, padded - r0);
        const int64_t valid = std::max<int64_t>(0, std::min(rows_out, a.tokens - r0));
        if (valid == 0) continue;  // never: r0 < tokens for every chunk of a padded range
        const void* xc = xs + r0 * a.xs_t * esz;
        hipLaunchKernelGGL(rowscale_kernel, dim3(blocks_of(valid * 64)), dim3(256), 0, s, xc, a.x_bf16, a.xs_t,
                           valid, cv.d, W.sc, W.nx, W.sig);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        RotArgs ra{};
        ra.x = xc;
        ra.ld = a.xs_t;
        ra.rows_valid = valid;
        ra.rows_out = rows_out;
        ra.d = cv.d;
        ra.sc = W.sc;
        ra.nx = W.nx;
        ra.sig = W.sig;
        ra.tiles = cv.rot_tiles + (cv.heads > 1 ? size_t(hh) * 2 * cv.d * cv.d : 0);
        ra.rec = rec + (r0 / kTile) * cv.tile_bytes;
        ra.tile_bytes = cv.tile_bytes;
        ra.off_nx = cv.off_nx;
        for (int t = 0; t < kMaxLevels - 1; ++t) ra.thr[t] = cv.uthr[t];
        for (int t = 0; t < kMaxLevels; ++t) ra.cen[t] = cv.ucen[t];
        ra.rhi = W.rhi;
        ra.rlo = W.rlo;
        ra.rr = W.rr;
        if ((e = launch_rotate(cv, prod ? 1 : 0, a.x_bf16 != 0, ra, s)) != hipSuccess) return e;
        if (prod) {
          SketchArgs sa{};
          sa.rhi = W.rhi;
          sa.rlo = W.rlo;
          sa.rows_valid = valid;
          sa.rows_out = rows_out;
          sa.m = cv.m;
          sa.tiles = cv.sk_tiles;
          sa.rec = ra.rec;
          sa.tile_bytes = cv.tile_bytes;
          sa.off_signs = cv.off_signs;
          sa.off_nr = cv.off_nr;
          sa.rr = W.rr;
          if ((e = launch_sketch(cv, 0, sa, s)) != hipSuccess) return e;
        }
      }
    }
  return hipSuccess;
}

namespace {
// query preparation scratch: per-row scales and norms, then the fp16 parts
// of sig q' handed to the sketch product
struct PrepWs {
  float *sc, *nx, *sig;
  uint16_t *rhi, *rlo;
};
size_t prep_ws(const CodecView& cv, int64_t nq, void* base, PrepWs* o) {
  const size_t R = size_t(nq), d = size_t(cv.d);
  auto rnd = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t sizes[5] = {rnd(R * 4), rnd(R * 4), rnd(R * 4), rnd(R * d * 2), rnd(R * d * 2)};
  size_t off[5], tot = 0;
  for (int i = 0; i < 5; ++i) { off[i] = tot; tot += sizes[i]; }
  if (o) {
    uint8_t* p = static_cast<uint8_t*>(base);
    o->sc = reinterpret_cast<float*>(p + off[0]);
    o->nx = reinterpret_cast<float*>(p + off[1]);
    o->sig = reinterpret_cast<float*>(p + off[2]);
    o->rhi = reinterpret_cast<uint16_t*>(p + off[3]);
    o->rlo = reinterpret_cast<uint16_t*>(p + off[4]);
  }
  return tot;
}
}  // namespace

size_t wide_query_prep_workspace(const CodecView& cv, int64_t nq) { return prep_ws(cv, nq, nullptr, nullptr); }

hipError_t launch_query_prep_wide(const CodecView& cv, const float* q, int64_t nq, float* qr, float* qs, void* ws,
                                  hipStream_t s) {
  PrepWs W;
  prep_ws(cv, nq, ws, &W);
  hipLaunchKernelGGL(rowscale_kernel, dim3(blocks_of(nq * 64)), dim3(256), 0, s, q, 0, int64_t(cv.d), nq, cv.d,
                     W.sc, W.nx, W.sig);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RotArgs ra{};
  ra.x = q;
  ra.ld = cv.d;
  ra.rows_valid = nq;
  ra.rows_out = nq;
  ra.d = cv.d;
  ra.sc = W.sc;
  ra.nx = W.nx;
  ra.sig = W.sig;
  ra.tiles = cv.rot_tiles;
  ra.rhi = W.rhi;
  ra.rlo = W.rlo;
  ra.yout = qr;
  if ((e = launch_rotate(cv, 2, false, ra, s)) != hipSuccess) return e;
  if (cv.mode != TQ_PROD) return hipSuccess;
  SketchArgs sa{};
  sa.rhi = W.rhi;
  sa.rlo = W.rlo;
  sa.rows_valid = nq;
  sa.rows_out = nq;
  sa.m = cv.m;
  sa.tiles = cv.sk_tiles;
  sa.sig = W.sig;
  sa.zout = qs;
  return launch_sketch(cv, 1, sa, s);
}

bool search_mfma_supported(const CodecView& cv) {
  return cv.layout == TQ_LAYOUT_ROW && cv.uniform && cv.heads == 1 && cv.d % 128 == 0 && cv.ubits >= 1 &&
         cv.ubits <= 3 && (cv.mode != TQ_PROD || cv.m == cv.d);
}

// 32-key blocks per wave of the search kernel (four would let each query
// fragment feed four MFMAs, but the accumulators then leave too few
// registers for the lists and the record chunks)
int search_nv(const CodecView&) { return 2; }

SearchPlan search_plan(const CodecView& cv, int64_t nq, int64_t n, int cus) {
  SearchPlan p{};
  p.nqb = int((nq + AR - 1) / AR);
  const int wgk = 128 * search_nv(cv);          // keys per workgroup tile
  const int64_t wgt = (n + wgk - 1) / wgk;      // workgroup tiles of keys
  int64_t ns = std::max<int64_t>(1, (int64_t(cus) + p.nqb - 1) / p.nqb);
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, wgt));
  ns = std::min<int64_t>(ns, 256);  // the merge takes at most 1024 lists per query
  p.nsplit = int(ns);
  p.keys_per_split = (wgt + ns - 1) / ns * wgk;
  p.nparts = 4 * p.nsplit;
  const int K = cv.d + (cv.mode == TQ_PROD ? cv.m : 0);
  auto rnd = [](size_t v) { return (v + 255) & ~size_t(255); };
  p.tiles_bytes = rnd(size_t(p.nqb) * AR * K * 2);
  p.inv_bytes = rnd(size_t(p.nqb) * AR * 4) * 2;  // query scales, then the shared thresholds
  return p;
}

hipError_t launch_search(const CodecView& cv, const float* qr, const float* qs, int64_t nq, const uint8_t* rec,
                         int64_t n, int k, const SearchPlan& p, void* tiles_ws, float* inv_ws, float* ps,
                         int64_t* pi, float* out_s, int64_t* out_i, float* dense, hipStream_t s) {
  if (!search_mfma_supported(cv) || (dense == nullptr && (k < 1 || k > 16)) || n >= (int64_t(1) << 31))
    return hipErrorNotSupported;
  const bool prod = cv.mode == TQ_PROD;
  const int m = prod ? cv.m : 0;
  uint16_t* tiles = static_cast<uint16_t*>(tiles_ws);
  // one-bit codes: the centroid (+-c) is folded into the query operand
  const float fc = cv.ubits == 1 ? cv.ucen[1] : 1.f;
  const float kq = prod ? kQjl / float(cv.m) : 0.f;
  const int64_t nrows = int64_t(p.nqb) * AR;
  hipLaunchKernelGGL(qtiles_kernel, dim3(blocks_of(nrows * 64)), dim3(256), 0, s, qr, qs, nq, nrows, cv.d, m, kq,
                     fc, tiles, inv_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SearchArgs sa{};
  sa.qtiles = tiles;
  sa.inv = inv_ws;
  sa.nq = nq;
  sa.nqb = p.nqb;
  sa.rec = rec;
  sa.n = n;
  sa.d = cv.d;
  sa.m = m;
  sa.tile_bytes = cv.tile_bytes;
  sa.off_signs = cv.off_signs;
  sa.off_nx = cv.off_nx;
  sa.off_nr = cv.off_nr;
  for (int t = 0; t < 8; ++t) sa.cen[t] = cv.ucen[t];
  sa.nsplit = p.nsplit;
  sa.keys_per_split = p.keys_per_split;
  sa.k = k;
  sa.nparts = p.nparts;
  sa.ps = ps;
  sa.pi = pi;
  sa.scores = dense;
  sa.thr = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(inv_ws) + p.inv_bytes / 2);
  if (!dense) {
    hipLaunchKernelGGL(fill_ord_kernel, dim3(blocks_of(nrows)), dim3(256), 0, s, sa.thr, nrows, -INFINITY);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 grid(unsigned(p.nqb * p.nsplit));
  // two waves per key block for 1 and 2 index bits; at 3 the centroid table
  // (32 KB) leaves no LDS for the second wave's transposition buffers
#define TQ_S(U, P, D, KM, NV, QW) \
  hipLaunchKernelGGL((search_kernel<U, P, D, KM, NV, QW>), grid, dim3(NT * QW), 0, s, sa)
#define TQ_S_UB(P, D, KM)                       \
  switch (cv.ubits) {                           \
    case 1: TQ_S(1, P, D, KM, 2, 2); break;     \
    case 2: TQ_S(2, P, D, KM, 2, 2); break;     \
    default: TQ_S(3, P, D, KM, 2, 1); break;    \
  }
  if (dense) {
    if (prod) { TQ_S_UB(true, true, 1) } else { TQ_S_UB(false, true, 1) }
    return hipGetLastError();
  }
  if (k <= 10) {
    if (prod) { TQ_S_UB(true, false, 10) } else { TQ_S_UB(false, false, 10) }
  } else {
    if (prod) { TQ_S_UB(true, false, 16) } else { TQ_S_UB(false, false, 16) }
  }
#undef TQ_S_UB
#undef TQ_S
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_topk_merge(ps, pi, nq, p.nparts, k, out_s, out_i, s);
}

}  // namespace tq
