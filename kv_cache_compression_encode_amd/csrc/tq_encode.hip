// Fused TurboQuant encode for d = 128 on CDNA4 (gfx950).
//
// One wavefront encodes one 64-vector record tile.  Per tile:
//   1. 128-bit loads of the input rows (lane = vector, half-wave = 64 coords),
//      n_x = ||x|| in fp32;
//   2. rotation Y^T = Pi X^T as 32x32x16 f16 MFMAs: 16 Pi is split into fp16
//      hi + lo parts (staged once per workgroup in LDS) and each input vector
//      is scaled by a power of two into the fp16 range (bf16 inputs are then
//      exact in fp16; fp32 inputs are split into hi + lo too), so y carries
//      ~2^-22 relative error, well inside the 1e-5 decision band even after
//      the sketch amplifies it by ||S_j|| ~ sqrt(m);
//   3. quantize: idx = #{t_k : t_k * n_x <= y_k * n_x} against the Lloyd-Max
//      boundaries (TurboQuant paper review, "Method"), codes packed as bit
//      planes (row layout: lane-local bits) or index-major col fields
//      (lanes OR-ed together by a butterfly, or a wavefront ballot at 1 bit);
//   4. prod: residual r = y - c[idx] kept in the MFMA accumulator layout, which
//      is exactly the B-operand layout of the next product, so the QJL sketch
//      Z^T = S R^T runs on MFMA without any transpose (S columns are permuted
//      once when staged); S is stored in fp16 and 32 r is split into fp16
//      hi + lo parts (two 32x32x16 f16 MFMAs, ~2^-22 relative); sign bits =
//      [z >= 0];
//   5. fp16 norms n_x and n_r = ||r||.
// The 32x32 accumulator of v_mfma_f32_32x32x16 holds, in lane l and register
// r, row 8*(r/4) + 4*(l/32) + r%4 and column l%32.
#include <hip/hip_runtime.h>

#include "tq_kernels.h"

namespace tq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int LDS_ROW = D + 8;  // 16-bit elements per staged row (16-byte pad)

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;

__device__ __forceinline__ f32x16 mfma32h(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t f16b(float x) {
  return uint32_t(__builtin_bit_cast(uint16_t, (_Float16)x));
}

// -1.0f in a scalar register the compiler cannot see through: fma(h, m1, x)
// with an fp16 h then stays one mixed-precision FMA (v_fma_mix_f32 reads the
// fp16 half in place) instead of being folded into a conversion plus a
// subtraction.
__device__ __forceinline__ float opaque_minus_one() {
  float m1;
  asm("s_mov_b32 %0, 0xbf800000" : "=s"(m1));
  return m1;
}

// Pack 8 floats into fp16 hi and lo fragments, x = hi + lo to ~2^-22
// relative: hi by a packed round-toward-zero conversion, the exact remainder
// x - hi rounded to nearest, each half by one mixed-precision FMA that reads
// its fp16 half of hi in place and writes its half of the lo word (mixlo,
// then mixhi into the same register: no separate packing step).
__device__ __forceinline__ uint32_t split_lo2(uint32_t hb, float v0, float v1) {
  uint32_t l;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %1, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(l)
      : "v"(hb), "v"(v0), "v"(v1));
  return l;
}
__device__ __forceinline__ void split8h(const float* v, u32x4& hi, u32x4& lo, float m1) {
  (void)m1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(v[2 * i], v[2 * i + 1]));
    hi[i] = h;
    lo[i] = split_lo2(h, v[2 * i], v[2 * i + 1]);
  }
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint32_t xor32(uint32_t v) {
  return __shfl_xor((int)v, 32, 64);
}
__device__ __forceinline__ float xor32f(float v) { return __shfl_xor(v, 32, 64); }

__device__ __forceinline__ uint16_t f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Output-row order of the rotation and sketch products.  LDS row
// 32b + 8a + 4h + c (a, c in 0..3, h in 0..1) holds matrix row 32b + 16h + 4a + c,
// so that accumulator register r of the lanes in half h of a 32x32 block holds
// coordinate 32b + 16h + r: each half-wave owns 16 consecutive coordinates and
// packs their bits with constant shifts.
__host__ __device__ constexpr int lds_row_of(int g) {
  return (g & ~31) | (((g >> 2) & 3) << 3) | (((g >> 4) & 1) << 2) | (g & 3);
}

// Stage N [128][128] 16-bit matrices into LDS rows of LDS_ROW elements,
// rows placed by lds_row_of; with colperm[m] bits 3 and 4 of the column
// index are swapped, matching the residual's register order in the sketch
// operand.  512 threads, 4 chunks of 16 bytes of each matrix per thread, in
// two phases: stage_load issues every load (one memory round trip for all
// N), stage_store writes LDS once they have arrived; loads issued between
// the two stay in flight across the stores.
// Next job of a workgroup's job counter in LDS: every lane of the wave adds
// (lane 0 one, the others zero), so that lane 0's return value is the
// counter before this wave's increment whatever order the lanes are served
// in.  Written as one LDS atomic with its wait: the compiler's own lowering
// of a wave-level atomic adds a loop over the active lanes and a branch.
__device__ __forceinline__ int take_job(int* counter, int lane) {
  const uint32_t addr = uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) int*)counter));
  const uint32_t one = lane == 0 ? 1u : 0u;
  uint32_t old;
  asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(old) : "v"(addr), "v"(one));
  return int(__builtin_amdgcn_readfirstlane(old));
}

constexpr int kStagePer = D * D / 8 / 512;
static_assert(D * D / 8 % 512 == 0, "whole chunks per thread");
template <int N>
__device__ __forceinline__ void stage_load(const uint16_t* const (&g)[N], u32x4 (&v)[N][kStagePer]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 0; m < N; ++m)
#pragma unroll
    for (int u = 0; u < kStagePer; ++u) v[m][u] = *reinterpret_cast<const u32x4*>(g[m] + (u * 512 + tid) * 8);
}
template <int N>
__device__ __forceinline__ void stage_store(uint16_t* const (&lds)[N], const bool (&colperm)[N],
                                            const u32x4 (&v)[N][kStagePer]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 0; m < N; ++m)
#pragma unroll
    for (int u = 0; u < kStagePer; ++u) {
      const int e = u * 512 + tid;
      const int row = e / (D / 8), col = (e % (D / 8)) * 8;
      const int c2 = colperm[m] ? ((col & ~24) | (((col >> 3) & 1) << 4) | (((col >> 4) & 1) << 3)) : col;
      *reinterpret_cast<u32x4*>(lds[m] + lds_row_of(row) * LDS_ROW + c2) = v[m][u];
    }
}


// Index of v among 2^UB Lloyd-Max cells: number of boundaries T[k] <= v, by
// a binary search of UB compares whose thresholds are picked with selects
// (ties go to the upper cell).  T holds 2^UB - 1 scaled boundaries.
typedef float f32x16v __attribute__((ext_vector_type(16)));

// Index of v among 2^UB Lloyd-Max cells: number of boundaries T[k] <= v, by
// a binary search of UB compares whose thresholds are picked with selects
// (ties go to the upper cell).  T holds the 2^UB - 1 scaled boundaries in a
// register vector (a plain array would be indexed through scratch memory).
template <int UB>
__device__ __forceinline__ int quant_tree(float v, f32x16v T) {
  if constexpr (UB == 1) {
    return v >= T[0] ? 1 : 0;
  } else if constexpr (UB == 2) {
    const bool b1 = v >= T[1];
    const bool b0 = v >= (b1 ? T[2] : T[0]);
    return (b1 ? 2 : 0) | (b0 ? 1 : 0);
  } else if constexpr (UB == 3) {
    const bool b2 = v >= T[3];
    const bool b1 = v >= (b2 ? T[5] : T[1]);
    const float t0 = b2 ? (b1 ? T[6] : T[4]) : (b1 ? T[2] : T[0]);
    const bool b0 = v >= t0;
    return (b2 ? 4 : 0) | (b1 ? 2 : 0) | (b0 ? 1 : 0);
  } else {
    static_assert(UB == 4, "1..4 index bits");
    const bool b3 = v >= T[7];
    const bool b2 = v >= (b3 ? T[11] : T[3]);
    const float t1 = b3 ? (b2 ? T[13] : T[9]) : (b2 ? T[5] : T[1]);
    const bool b1 = v >= t1;
    const float u0 = b2 ? (b1 ? T[14] : T[12]) : (b1 ? T[10] : T[8]);
    const float u1 = b2 ? (b1 ? T[6] : T[4]) : (b1 ? T[2] : T[0]);
    const bool b0 = v >= (b3 ? u0 : u1);
    return (b3 ? 8 : 0) | (b2 ? 4 : 0) | (b1 ? 2 : 0) | (b0 ? 1 : 0);
  }
}

// Same search, returning the index bits b[p] (bit p of the index) and the
// selected level of `L` (2^UB values) without building the index as an
// integer: the level is picked by selects on the bits, most significant first.
template <int UB>
__device__ __forceinline__ float quant_bits(float v, f32x16v T, const float* L, bool (&b)[4]) {
  if constexpr (UB == 1) {
    b[0] = v >= T[0];
    return b[0] ? L[1] : L[0];
  } else if constexpr (UB == 2) {
    b[1] = v >= T[1];
    b[0] = v >= (b[1] ? T[2] : T[0]);
    const float hi = b[1] ? L[3] : L[1], lo = b[1] ? L[2] : L[0];
    return b[0] ? hi : lo;
  } else if constexpr (UB == 3) {
    b[2] = v >= T[3];
    b[1] = v >= (b[2] ? T[5] : T[1]);
    b[0] = v >= (b[2] ? (b[1] ? T[6] : T[4]) : (b[1] ? T[2] : T[0]));
    const float l3 = b[2] ? (b[1] ? L[7] : L[5]) : (b[1] ? L[3] : L[1]);
    const float l2 = b[2] ? (b[1] ? L[6] : L[4]) : (b[1] ? L[2] : L[0]);
    return b[0] ? l3 : l2;
  } else {
    static_assert(UB == 4, "1..4 index bits");
    b[3] = v >= T[7];
    b[2] = v >= (b[3] ? T[11] : T[3]);
    b[1] = v >= (b[3] ? (b[2] ? T[13] : T[9]) : (b[2] ? T[5] : T[1]));
    const float u0 = b[2] ? (b[1] ? T[14] : T[12]) : (b[1] ? T[10] : T[8]);
    const float u1 = b[2] ? (b[1] ? T[6] : T[4]) : (b[1] ? T[2] : T[0]);
    b[0] = v >= (b[3] ? u0 : u1);
    float l[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) l[k] = L[k];
#pragma unroll
    for (int bt = 3; bt >= 0; --bt) {
      const int half = 1 << bt;
#pragma unroll
      for (int k = 0; k < half; ++k) l[k] = b[bt] ? l[k + half] : l[k];
    }
    return l[0];
  }
}

// The uniform codebooks are Lloyd-Max solutions for a symmetric law, so
// their boundaries are symmetric about 0 (T[L/2 - 1] = 0, T[L/2 - 1 + k] =
// -T[L/2 - 1 - k]) and so are their levels.  The 4-level quantizer below
// uses this: the sign of v picks the half and |v| is compared with the one
// positive boundary.  Decisions equal those of the full search except when
// v < 0 lies exactly on a boundary (a tie, which then goes to the lower cell).
// 16-level col codes instead look their coordinate's bucket up in a table of
// the boundaries and make one compare in bucket units (see the kernels).

// Transpose of an 8 x 8 matrix of nibbles held by 8 consecutive lanes (lane
// t of the group holds row t, element c at bits 4c..4c+3): on return lane t
// holds column t.  Three exchange stages with the lanes 4, 2 and 1 away swap
// blocks of 4, 2 and 1 nibbles; the per-lane selectors come from
// nib_transpose_consts.
struct NibT {
  uint32_t selA, selB, rotC, mskC;
};
__device__ __forceinline__ NibT nib_transpose_consts(int t) {
  NibT c;
  c.selA = (t & 4) ? 0x03020706u : 0x05040100u;  // own bytes 0,1 + partner's 0,1 / partner's 2,3 + own 2,3
  c.selB = (t & 2) ? 0x03070105u : 0x06020400u;  // interleave bytes with the partner's
  c.rotC = (t & 1) ? 4u : 28u;                    // partner's nibbles to the other half of each byte
  c.mskC = (t & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;   // nibbles kept from the own word
  return c;
}
__device__ __forceinline__ uint32_t nib_transpose8(uint32_t w, const NibT& c) {
  uint32_t x = uint32_t(__builtin_amdgcn_ds_swizzle(int(w), 0x101F));  // lane ^ 4 (bitmask mode, xor 4)
  w = __builtin_amdgcn_perm(x, w, c.selA);
  x = uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]: lane ^ 2
  w = __builtin_amdgcn_perm(x, w, c.selB);
  x = uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]: lane ^ 1
  x = __builtin_amdgcn_alignbit(x, x, c.rotC);
  return (w & c.mskC) | (x & ~c.mskC);
}

// w = 2 w + [b]: one v_addc with the comparison's lane mask as the carry in
// (the mask is the same SGPR pair the selects of the quantizer use).  Bits
// pushed for registers r = 15 .. 0 land at bit r.
__device__ __forceinline__ uint32_t push_bit(uint32_t w, bool b) {
  const uint64_t m = __ballot(b);
  uint32_t r;
  uint64_t cout;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(cout) : "v"(w), "s"(m));
  (void)cout;
  return r;
}

// w = 2 w + (bit of this lane in the lane mask m), one v_addc.
__device__ __forceinline__ uint32_t push_mask(uint32_t w, uint64_t m) {
  uint32_t r;
  uint64_t cout;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(cout) : "v"(w), "s"(m));
  (void)cout;
  return r;
}

// 4 levels: P = T[2] scaled like v, L2 / L3 levels 2 / 3 (levels 0 / 1 are
// their negatives), L2, L3 > 0.  Index bit 1 is [v >= 0] and index bit 0 is
// [v >= 0] == [|v| >= P].  Appends the sign bit of v ([v < 0]) to w1 and
// [|v| >= P] to w0 (one v_alignbit and one v_addc); sym2_finish turns the
// two words into the index planes once all bits are in.  Returns the
// selected level.  v is never -0 here (accumulator values).
__device__ __forceinline__ float quant2_sym_push(float v, float P, float L2, float L3, uint32_t& w0,
                                                 uint32_t& w1) {
  const bool m = fabsf(v) >= P;
  w0 = push_mask(w0, __ballot(m));
  w1 = __builtin_amdgcn_alignbit(w1, __float_as_uint(v), 31);
  // the level with the sign of v, formed on the bits (one v_and_or) so that
  // the caller's -level stays a source modifier of its FMA
  return __uint_as_float(__float_as_uint(m ? L3 : L2) | (__float_as_uint(v) & 0x80000000u));
}
// After quant2_sym_push over the bits in `mask`: w1 = [v < 0] bits and
// w0 = [|v| >= P] bits become index bit 0 = [v < 0] xor [|v| >= P] and
// index bit 1 = not [v < 0].
__device__ __forceinline__ void sym2_finish(uint32_t& w0, uint32_t& w1, uint32_t mask) {
  w0 ^= w1;
  w1 ^= mask;
}

// Sign word of 16 accumulator values, pushed from register 15 down to 0:
// bit r = [z_r >= 0].  The float sign bits are shifted in (one v_alignbit
// each) and flipped at the end; z is never -0 (each MFMA chain starts at +0
// and a sum with +0 never rounds to -0).
__device__ __forceinline__ uint32_t sign_word16(const f32x16& z) {
  uint32_t neg = 0u;
#pragma unroll
  for (int r = 15; r >= 0; --r) neg = __builtin_amdgcn_alignbit(neg, __float_as_uint(z[r]), 31);
  return neg ^ 0xffffu;
}

// OR across groups of `VPD` consecutive lanes (8 or 16) with DPP moves:
// quad xor-1, quad xor-2, then half-row / row mirrors.
template <int VPD>
__device__ __forceinline__ uint32_t group_or(uint32_t w) {
  w |= uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  w |= uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  if constexpr (VPD >= 8) w |= uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0x141, 0xF, 0xF, true));  // row_half_mirror
  if constexpr (VPD >= 16) w |= uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0x140, 0xF, 0xF, true)); // row_mirror
  return w;
}

// Encode of the tiles of one workgroup: workgroup bx of the gx that share
// the (sequence, head) set bh.  The kernels below call it with their grid
// coordinates.
template <int NB, bool BF16IN, int MODE, bool COL, bool UNIFORM, int UB, int SPLIT = 0>
__device__ __forceinline__ void encode_d128_body(const CodecView& cv, const EncodeArgs& a, const int bx,
                                                 const int gx, const int64_t bh) {
  // MODE: 0 mse, 1 prod with a full 128-dim MFMA sketch, 2 prod with a small
  // (m <= 4) sketch on rotated dims 0..m-1 (SpectralQuant selective QJL).
  // SPLIT: outlier-channel split codec in stored order, each group
  // normalised by its own norm, summed over its channels (the head's channel
  // mask) as the rows are loaded.  SPLIT 1: 32 outlier coordinates (half 0,
  // registers 0..7 of every 32-dim block) at 2 index bits and 96 regular ones
  // at 1 bit, with symmetric searches and plane words; SPLIT 2: any outlier
  // count o (o / 4 = o4 leading coordinates of every 32-dim block) and index
  // bits, per-dim binary searches against the group codebooks in LDS, the
  // bits written plane by plane as byte runs of the row bit string.
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* sPiHi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sPiLo = sPiHi + D * LDS_ROW;
  uint16_t* sSk = sPiLo + D * LDS_ROW;  // S is stored in fp16 (exact, no low part)
  float* sThr = reinterpret_cast<float*>(MODE == 1 ? (uint8_t*)(sSk + D * LDS_ROW)
                                                   : (uint8_t*)sSk);
  float* sCen = sThr + D * kMaxLevels;
  // 16-level COL codes: bucket table of the boundaries (one compare per coordinate)
  __shared__ float2 sQ[UNIFORM && COL && UB == 4 && MODE == 0 ? kQMax : 1];

  if (bh >= a.batch * a.heads) return;
  const int64_t b = bh / a.heads, h = bh % a.heads;
  const int hc = cv.heads > 1 ? int(h) : 0;

  const int lane = lane_id();
  const int j = lane & 31, hh = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int64_t ntiles = (a.tokens + kTile - 1) / kTile;
  const uint8_t* xbase = static_cast<const uint8_t*>(a.x) +
                         (b * a.xs_b + h * a.xs_h) * (BF16IN ? 2 : 4);
  uint8_t* rbase = a.rec + b * a.rs_b + h * a.rs_h;

  constexpr int NSUB = 2 / NB;            // sub-tiles of 32*NB vectors per tile
  constexpr int NPL = UNIFORM ? UB : 1;   // planes held in the word arrays
  constexpr int LV = 1 << (UNIFORM ? UB : 1);
  // symmetric search paths: 16-level col codes (values), 4-level row codes
  constexpr bool SYM4 = UNIFORM && COL && UB == 4 && MODE == 0;
  constexpr bool SYM2 = UNIFORM && !COL && UB == 2;
  // blocks software-pipelined (two rotation accumulators live at once)
  constexpr bool PIPE = (SYM4 || (SYM2 && MODE == 1)) && NB == 1 && SPLIT == 0 && BF16IN;
  // SpectralQuant key structure (non-uniform, MODE 2, UB = 2): dims 0..3 carry
  // 1..5 bits, every other dim one bit
  constexpr bool SQK = !UNIFORM && !SPLIT && MODE == 2 && UB == 2;
  const NibT nibc = nib_transpose_consts(int(threadIdx.x & 7));

  const int nwaves = blockDim.x >> 6;
  const int64_t tstep = int64_t(gx) * nwaves;
  // bf16 input: the raw rows of the next sub-tile are loaded while the
  // current one is processed (register double buffer).
  // Loads are unconditional (rows past the end read the last row instead and
  // their results are discarded), so no load sits behind a branch and the
  // wait counters stay exact across the prefetch.
  // The raw rows alternate between two register sets (the next sub-tile's
  // loads go to one set while the other is processed; no copies between them).
  u32x4 bufA[NB][8], bufB[NB][8];
  auto load_raw = [&](int64_t tl, int sb, u32x4 (&dst)[NB][8]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int64_t t = tl * kTile + sb * 32 * NB + nb * 32 + j;
      const int64_t tc = (tl < ntiles && t < a.tokens) ? t : a.tokens - 1;
      const uint16_t* row = reinterpret_cast<const uint16_t*>(xbase) + tc * a.xs_t + 64 * hh;
#pragma unroll
      for (int c = 0; c < 8; ++c) dst[nb][c] = *reinterpret_cast<const u32x4*>(row + 8 * c);
    }
  };
  auto process = [&](const u32x4 (&cur)[NB][8], int64_t tile, int sub) {
    uint8_t* trec = rbase + tile * cv.tile_bytes;
    const float m1 = opaque_minus_one();
    {
      // ---------------------------------------------------------- load X
      // xh/xl: fp16 hi/lo fragments of x * 2^e, e chosen per vector so that
      // max|x| * 2^e lies in [2^14, 2^15); w = 16 * 2^e * s_x is the factor
      // between the accumulator and the rotated unit vector y.
      u32x4 xh[NB][8], xl[NB][8];
      float sx[NB], nxv[NB], wsc[NB];
      // norms are sqrt(sum of squares) / nd: nd = 1 when the squares were
      // summed unscaled, 2^e when they were summed over x * 2^e (then no
      // square underflows, whatever the vector's magnitude)
      float nd[NB];
      float so2[NB];  // SPLIT: sum of squares over this vector's outlier channels
      // SPLIT: outlier boundary t_2 and levels c_2, c_3 (dim 0), regular
      // level c_1 (dim 8), and this half's outlier-channel mask (channels
      // 64 hh ..); read here, per tile, so that they stay in registers
      float spl_t2 = 0.f, spl_c2 = 0.f, spl_c3 = 0.f, spl_c1 = 0.f, spl_lo = 0.f, spl_hi = 0.f;
      uint32_t om[2] = {0u, 0u};
      if constexpr (SPLIT != 0) {
        om[0] = cv.omask[hc * 4 + 2 * hh];
        om[1] = cv.omask[hc * 4 + 2 * hh + 1];
      }
      if constexpr (SPLIT == 1) {
        const float* th = cv.thr + size_t(hc) * D * kMaxLevels;
        const float* ce = cv.cen + size_t(hc) * D * kMaxLevels;
        spl_t2 = th[2];
        spl_c2 = 32.f * ce[2];
        spl_c3 = 32.f * ce[3];
        spl_c1 = 32.f * ce[8 * kMaxLevels + 1];
        spl_lo = hh ? spl_c1 : spl_c2;  // level magnitude below / above t_2
        spl_hi = hh ? spl_c1 : spl_c3;  // (half 1: the regular level)
      }
      bool valid[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int slot = sub * 32 * NB + nb * 32 + j;
        const int64_t t = tile * kTile + slot;
        valid[nb] = t < a.tokens;
        nd[nb] = 1.f;
        float ss = 0.f, mx = 0.f;
        if (BF16IN) {
          // raw bf16 pairs (prefetched) stay packed until the scale is known
          const u32x4* r = cur[nb];
          if constexpr (!SPLIT) {
            // ||x||^2 by bf16 dot products of each word with itself (the
            // products are exact in fp32), four chains; the words go through
            // scalars (a bit cast straight from a vector element has read
            // element 0)
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t w = r[c][i];
                const bf2_t h = __builtin_bit_cast(bf2_t, w);
                s4[i] = __builtin_amdgcn_fdot2_f32_bf16(h, h, s4[i], false);
              }
            ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
          } else {
            // two chains; the squares of bf16 values are exact in fp32
            float s0 = 0.f, s1 = 0.f;
            float o0 = 0.f, o1 = 0.f;  // outlier channels only
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(r[c][i] << 16), hi = __uint_as_float(r[c][i] & 0xffff0000u);
                {
                  // channel 64 hh + 8c + 2i (+1): bit (8c + 2i) % 32 of mask word c / 4
                  const int k = (8 * c + 2 * i) & 31;
                  const uint32_t lw = r[c][i] << 16, hw = r[c][i] & 0xffff0000u;
                  const float lo_o = __uint_as_float(lw & uint32_t(-int((om[c >> 2] >> k) & 1u)));
                  const float hi_o = __uint_as_float(hw & uint32_t(-int((om[c >> 2] >> (k + 1)) & 1u)));
                  o0 = fmaf(lo_o, lo_o, o0);
                  o1 = fmaf(hi_o, hi_o, o1);
                  const float lo_r = lo - lo_o, hi_r = hi - hi_o;  // exact: x or 0
                  s0 = fmaf(lo_r, lo_r, s0);
                  s1 = fmaf(hi_r, hi_r, s1);
                }
              }
            ss = s0 + s1;
            so2[nb] = o0 + o1;
          }
          if constexpr (SPLIT) {
            // ss holds the regular channels here; the scale below needs ||x||
            ss += xor32f(ss);
            so2[nb] += xor32f(so2[nb]);
            nxv[nb] = sqrtf(ss);        // regular instance's norm
            ss += so2[nb];
          } else {
            ss += xor32f(ss);
          }
          // scale 2^s, s = 14 - floor(log2 ||x||): every |x_i| 2^s < 2^15.
          // x_i 2^s in fp16 is then formed from the bf16 bits directly: the
          // exponent field drops by D = 112 - s (saturating at 0, which
          // flushes elements below 2^-14 of the scaled range, i.e. under
          // 2^-28 ||x||), the 7 mantissa bits move up by 3, the sign stays.
          // Norms whose floor(log2) is below -50 (their squares may be
          // denormal or flushed: zero vectors too), and non-finite ones, take
          // the general path below (float scaling by the largest element,
          // squares summed over the scaled values).
          const int es = int((__float_as_uint(ss) >> 23) & 0xff);  // biased exponent of ||x||^2
          const int en = (es - 127) >> 1;                            // floor(log2 ||x||) (normal ss)
          const bool fast = es > 0 && es < 255 && en >= -50;
          if (__builtin_expect(__ballot(!fast) == 0, 1)) {
            const int dsh = 98 + en;  // D
            const uint32_t dd = uint32_t(dsh) << 7;
            const u16x2 sub2 = {uint16_t(dd), uint16_t(dd)};
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t w = r[c][i];
                u16x2 e = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
                e = __builtin_elementwise_sub_sat(e, sub2);
                e = e << u16x2{3, 3};
                xh[nb][c][i] = (w & 0x80008000u) | __builtin_bit_cast(uint32_t, e);
              }
            const float p2 = __uint_as_float(uint32_t(141 - en) << 23);
            wsc[nb] = 16.f * p2;
          } else {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(r[c][i] << 16), hi = __uint_as_float(r[c][i] & 0xffff0000u);
                mx = fmaxf(mx, fmaxf(fabsf(lo), fabsf(hi)));
              }
            mx = fmaxf(mx, xor32f(mx));
            const int ebits = int((__float_as_uint(mx) >> 23) & 0xff);
            const float p2 = mx > 0.f ? __uint_as_float(uint32_t(min(254, max(1, 268 - ebits))) << 23) : 1.f;
            // x * 2^e is exact in fp16 (8 significant bits, exponent in range)
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(r[c][i] << 16) * p2;
                const float hi = __uint_as_float(r[c][i] & 0xffff0000u) * p2;
                xh[nb][c][i] = f16b(lo) | (f16b(hi) << 16);
              }
            // squares of the scaled values (none underflows), from the row in
            // memory again: a rare path, kept as a short loop
            const int64_t tr = valid[nb] ? t : a.tokens - 1;
            const uint16_t* xrow = reinterpret_cast<const uint16_t*>(xbase) + tr * a.xs_t + 64 * hh;
            float tt = 0.f, uu = 0.f;  // SPLIT: uu sums the outlier channels
#pragma unroll 1
            for (int e = 0; e < 64; ++e) {
              const float xe = __uint_as_float(uint32_t(xrow[e]) << 16) * p2;
              bool ob = false;
              if constexpr (SPLIT) ob = ((e < 32 ? om[0] : om[1]) >> (e & 31)) & 1u;
              uu = fmaf(ob ? xe : 0.f, xe, uu);
              tt = fmaf(ob ? 0.f : xe, xe, tt);
            }
            tt += xor32f(tt);
            nd[nb] = p2;
            if constexpr (SPLIT) {
              uu += xor32f(uu);
              nxv[nb] = sqrtf(tt) / p2;  // regular instance's norm
              so2[nb] = uu;              // outliers, scaled
            } else {
              ss = tt;
            }
            wsc[nb] = 16.f * p2;
          }
        } else {
          const int64_t tc = valid[nb] ? t : a.tokens - 1;  // unconditional load, see load_raw
          const float* row = reinterpret_cast<const float*>(xbase) + tc * a.xs_t + 64 * hh;
          float v[8][8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float4 p0 = *reinterpret_cast<const float4*>(row + 8 * c);
            const float4 p1 = *reinterpret_cast<const float4*>(row + 8 * c + 4);
            v[c][0] = p0.x; v[c][1] = p0.y; v[c][2] = p0.z; v[c][3] = p0.w;
            v[c][4] = p1.x; v[c][5] = p1.y; v[c][6] = p1.z; v[c][7] = p1.w;
          }
#pragma unroll
          for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[c][i]));
          mx = fmaxf(mx, xor32f(mx));
          // 2^(14 - floor(log2 mx)) from the exponent field of mx
          const int ebits = int((__float_as_uint(mx) >> 23) & 0xff);
          const float p2 = mx > 0.f ? __uint_as_float(uint32_t(min(254, max(1, 268 - ebits))) << 23) : 1.f;
          // squares summed over the scaled values (none underflows)
          float so = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            float sc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              sc[i] = v[c][i] * p2;
              if constexpr (SPLIT) {
                const bool ob = (om[c >> 2] >> ((8 * c + i) & 31)) & 1u;
                so = fmaf(ob ? sc[i] : 0.f, sc[i], so);
                ss = fmaf(ob ? 0.f : sc[i], sc[i], ss);
              } else {
                ss = fmaf(sc[i], sc[i], ss);
              }
            }
            split8h(sc, xh[nb][c], xl[nb][c], m1);
          }
          ss += xor32f(ss);
          nd[nb] = p2;
          if constexpr (SPLIT) {
            so += xor32f(so);
            so2[nb] = so;                 // outliers, scaled
            nxv[nb] = sqrtf(ss) / p2;     // regular instance's norm
          }
          wsc[nb] = 16.f * p2;
        }
        if constexpr (!SPLIT) {
          nxv[nb] = sqrtf(ss) / nd[nb];
          // A zero vector encodes y = 0: thresholds and residual in unit scale.
          sx[nb] = nxv[nb] > 0.f ? nxv[nb] : 1.f;
          wsc[nb] *= sx[nb];
        }
      }

      // boundaries scaled to the accumulator (uniform codec); prod: the
      // residual is formed directly in unit scale times 32, rsd = v rs - 32 c
      f32x16v T[NB];
      float sK[NB];  // SYM4: bucket units per accumulator unit
      float rs[NB];
      float C32[LV];
      if (UNIFORM) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int k = 0; k < LV - 1; ++k) T[nb][k] = cv.uthr[k] * wsc[nb];
          if (SYM4) sK[nb] = cv.qinvw / wsc[nb];
          rs[nb] = 32.f / wsc[nb];
        }
#pragma unroll
        for (int k = 0; k < LV; ++k) C32[k] = 32.f * cv.ucen[k];
      }

      uint32_t cw[NB][NPL];      // code bits of the current 32-dim block (this half's 16), plane p
      uint32_t gw[NB][SPLIT == 2 ? kMaxBits : 1];  // SPLIT 2: plane p bits of this half's 16 coordinates
      uint32_t tailw[NB];        // non-uniform row layout: bits beyond plane 0
      uint32_t sw[NB][4];        // sign bits (row layout), this half's 16 per word
      float rr[NB];
      f32x16 z[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        rr[nb] = 0.f;
        tailw[nb] = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sw[nb][q] = 0;
          if (MODE == 1) z[nb][q] = f32x16{};
        }
      }
      float zsmall[NB][4];
      float rsmall[NB][4];
      // SPLIT: per group the factor between the accumulator and the unit
      // vector (16 2^e times the group's norm; a zero group encodes y = 0)
      float nxo[NB], rso[NB], rsr[NB], rro[NB], P2o[NB], wso_[NB], wsr_[NB];
      uint32_t p1w[NB];
      if constexpr (SPLIT != 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          nxo[nb] = sqrtf(so2[nb]) / nd[nb];
          const float wso = wsc[nb] * (nxo[nb] > 0.f ? nxo[nb] : 1.f);
          const float wsr = wsc[nb] * (nxv[nb] > 0.f ? nxv[nb] : 1.f);
          wso_[nb] = wso;
          wsr_[nb] = wsr;
          rso[nb] = 32.f / wso;
          rsr[nb] = 32.f / wsr;
          P2o[nb] = hh ? -INFINITY : spl_t2 * wso;  // half 1 holds no outliers
          rro[nb] = 0.f;
          p1w[nb] = 0u;
        }
      }
      // 2.5-bit split values (col records): the 7 outlier boundaries (3 index
      // bits, stored dim 0) and the 3 regular ones (2 bits, stored dim 8),
      // scaled to the accumulator by each group's factor, in registers
      constexpr bool SCOL = SPLIT == 2 && COL && MODE == 0;
      f32x16v Tso[NB], Tsr[NB];
      if constexpr (SCOL) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int k = 0; k < 7; ++k) Tso[nb][k] = sThr[k] * wso_[nb];
#pragma unroll
          for (int k = 0; k < 3; ++k) Tsr[nb][k] = sThr[8 * kMaxLevels + k] * wsr_[nb];
        }
      }

      // ------------------------------------------------ rotation block
      // one accumulation chain per 32-vector block: Pi_hi x_hi, Pi_lo x_hi
      // (and Pi_hi x_lo for fp32 input); register r of half hh holds
      // coordinate 32 mb + 16 hh + r
      auto rotate = [&](int mb, f32x16 (&acc)[NB]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
        // the Pi fragments are read from LDS two steps ahead of the MFMAs
        // that take them, so that the LDS latency overlaps the chain
        // (one step ahead in the software pipeline, where the quantization
        // of the previous block fills the wait)
        constexpr int RD = PIPE ? 2 : 3;
        u32x4 fh[RD], fl[RD];
        auto read_pi = [&](int c) {
          const int off = (32 * mb + j) * LDS_ROW + 64 * hh + 8 * c;
          fh[c % RD] = *reinterpret_cast<const u32x4*>(sPiHi + off);
          fl[c % RD] = *reinterpret_cast<const u32x4*>(sPiLo + off);
        };
#pragma unroll
        for (int c = 0; c < RD - 1; ++c) read_pi(c);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (c + RD - 1 < 8) read_pi(c + RD - 1);
          const u32x4 ah = fh[c % RD], al = fl[c % RD];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            acc[nb] = mfma32h(ah, xh[nb][c], acc[nb]);
            acc[nb] = mfma32h(al, xh[nb][c], acc[nb]);
            if (!BF16IN) acc[nb] = mfma32h(ah, xl[nb][c], acc[nb]);
          }
        }
      };
      // quantize, pack and sketch block mb from its rotated coordinates
      auto block = [&](int mb, f32x16 (&acc)[NB]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int p = 0; p < NPL; ++p) cw[nb][p] = 0;
        if constexpr (SPLIT == 2)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int p = 0; p < kMaxBits; ++p) gw[nb][p] = 0;
        // ------------------------------------------------ quantize block
        uint32_t colkeep[NB][2];
        uint32_t pk[NB][2];  // SYM4: nibbles of registers 8k .. 8k + 7 (register 8k + c at bits 4c)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int r = 15; r >= 0; --r) {  // descending: row-code bits are pushed MSB first
            const int dim = 32 * mb + 16 * hh + r;
            const float v = acc[nb][r];
            int idx = 0;
            float chat = 0.f;
            if constexpr (SPLIT == 1) {
              // registers 0..7 of half 0: outlier, 2 index bits (symmetric
              // 4-level search: bit 1 = [v >= 0], bit 0 = [v >= 0] == [|v| >= t_2]);
              // all others: regular, 1 bit = [v >= 0] (2 symmetric levels).
              // Each pushed bit is the complement of the index bit (flipped
              // per word after the block): the sign bit of v (never -0), or for
              // the outliers' bit 0 the sign bit of v xor (|v| - t_2), since
              // [v < 0] xor [|v| < t_2] = not ([v >= 0] == [|v| >= t_2]).  On
              // half 1, P2o = -inf makes |v| - P2o positive, so registers 0..7
              // push the sign bit of v there too.
              const uint32_t vb = __float_as_uint(v);
              if (r < 8) {
                const float u = fabsf(v) - P2o[nb];
                cw[nb][0] = __builtin_amdgcn_alignbit(cw[nb][0], vb ^ __float_as_uint(u), 31);
                p1w[nb] = __builtin_amdgcn_alignbit(p1w[nb], vb, 31);  // plane 1 (kept from half 0)
                const float c = u >= 0.f ? spl_hi : spl_lo;
                chat = __uint_as_float(__float_as_uint(c) | (vb & 0x80000000u));
              } else {
                cw[nb][0] = __builtin_amdgcn_alignbit(cw[nb][0], vb, 31);
                chat = __uint_as_float(__float_as_uint(spl_c1) | (vb & 0x80000000u));
              }
            } else if constexpr (SCOL) {
              // idx = #{t_k <= y} by the register search of the coordinate's
              // group (the same products t_k w as the general search below)
              const bool og = 16 * hh + r < cv.o4;
              const int io = quant_tree<3>(v, Tso[nb]), ir = quant_tree<2>(v, Tsr[nb]);
              idx = og ? io : ir;
            } else if constexpr (SPLIT == 2) {
              // the coordinate's group codebook (boundaries +inf past its
              // levels), against the group's scale: idx = #{t_k <= y}
              const bool og = 16 * hh + r < cv.o4;
              const float wg = og ? wso_[nb] : wsr_[nb];
              const float* Tt = sThr + dim * kMaxLevels;
              int k = 0;
#pragma unroll
              for (int st = 16; st >= 1; st >>= 1) k += v >= Tt[k + st - 1] * wg ? st : 0;
              idx = k;
              chat = 32.f * sCen[dim * kMaxLevels + k];
            } else if (UNIFORM && !COL) {
              // row layout: the index bits go straight into the plane words
              if constexpr (SYM2) {
                chat = quant2_sym_push(v, T[nb][2], C32[2], C32[3], cw[nb][0], cw[nb][NPL - 1]);
              } else {
                bool bits[4] = {false, false, false, false};
                chat = quant_bits<UB>(v, T[nb], C32, bits);
#pragma unroll
                for (int p = 0; p < NPL; ++p) cw[nb][p] = push_bit(cw[nb][p], bits[p]);
              }
            } else if (SYM4) {
              // bucket of y, clamped to the table by one median-of-three
              // (a NaN that survives it converts to bucket 0), then one
              // compare against the bucket's boundary: the index is the
              // count of boundaries below the bucket, plus one at or above
              // its boundary
              const float u = __builtin_amdgcn_fmed3f(fmaf(v, sK[nb], cv.qoff), 0.f, float(cv.qn - 1));
              const float2 e = sQ[uint32_t(u)];
              const uint32_t w0 = (r & 7) == 7 ? 0u : pk[nb][r >> 3];
              pk[nb][r >> 3] = (w0 << 4) + uint32_t(__float_as_int(e.y)) + (u >= e.x ? 1u : 0u);
            } else if (UNIFORM) {
              idx = quant_tree<UB>(v, T[nb]);
              if (MODE != 0) {
                // select tree over the (32x) centroids driven by the index bits
                float lvl[LV];
#pragma unroll
                for (int k = 0; k < LV; ++k) lvl[k] = C32[k];
#pragma unroll
                for (int bt = 0; bt < UB; ++bt) {
                  const bool on = (idx >> bt) & 1;
#pragma unroll
                  for (int k = 0; k < (LV >> (bt + 1)); ++k) lvl[k] = on ? lvl[2 * k + 1] : lvl[2 * k];
                }
                chat = lvl[0];
              }
            } else if constexpr (SQK) {
              if (mb == 0 && r < 4) {
                // dims 0..3 (half 0) and 16..19 (half 1): branch-free binary
                // search over the dim's 31 boundaries (unused ones are +inf),
                // idx = number of boundaries <= v
                const float* Tt = sThr + dim * kMaxLevels;
                int k = 0;
#pragma unroll
                for (int st = 16; st >= 1; st >>= 1) k += v >= Tt[k + st - 1] * wsc[nb] ? st : 0;
                idx = k;
                chat = sCen[dim * kMaxLevels + k] * wsc[nb];
              } else {
                // one bit on every other dim: the 2-level boundary is 0, so the
                // code is the sign; no level is needed (the residual covers
                // dims < 4 only)
                idx = v >= 0.f ? 1 : 0;
              }
            } else {
              const int L = 1 << cv.dim_bits[dim];
              chat = sCen[dim * kMaxLevels] * wsc[nb];
              for (int k = 0; k < L - 1; ++k) {
                const bool ge = v >= sThr[dim * kMaxLevels + k] * wsc[nb];
                idx += ge ? 1 : 0;
                chat = ge ? sCen[dim * kMaxLevels + k + 1] * wsc[nb] : chat;
              }
            }
            if (!valid[nb]) idx = 0;
            if (!COL) {
              if (SQK) {
                cw[nb][0] |= uint32_t(idx & 1) << r;
                if (mb == 0 && r < 4) {
                  // bits 1.. of dims 0..3 into the tail (half 1's dims have none)
#pragma unroll
                  for (int p = 1; p < kMaxBits; ++p) {
                    const int pos = cv.bitpos[p * D + dim];
                    const uint32_t bit = pos >= 0 ? uint32_t((idx >> p) & 1) : 0u;
                    tailw[nb] |= bit << (pos >= 0 ? pos - D : 0);
                  }
                }
              } else if constexpr (SPLIT == 2) {
#pragma unroll
                for (int p = 0; p < kMaxBits; ++p) gw[nb][p] |= uint32_t((idx >> p) & 1) << r;
              } else if (!UNIFORM && !SPLIT) {
                cw[nb][0] |= uint32_t(idx & 1) << r;
                for (int p = 1; p < kMaxBits; ++p) {
                  const int pos = cv.bitpos[p * D + dim];
                  if (pos >= 0) tailw[nb] |= uint32_t((idx >> p) & 1) << (pos - D);
                }
              }
            } else if constexpr (SPLIT == 2) {
              // split values in col records (32 outlier coordinates at 3
              // index bits, the others at 2): the 8 tokens of a group (8
              // consecutive lanes) form one word of b-bit codes, stored as b
              // bytes in slot vb = dim / 16 of lane block n = dim % 16 of the
              // group (block n < 8: 3- and 2-byte slots alternating, 20
              // bytes; n >= 8: 2-byte slots, 16 bytes; 288 bytes a group)
              const bool og = (16 * hh + r) < cv.o4;
              const int b = og ? 3 : 2;
              const uint32_t w = group_or<8>(uint32_t(idx) << (b * (j & 7)));
              const int n = dim & 15, vb = dim >> 4;
              const int off = n < 8 ? 20 * n + 5 * (vb >> 1) + 3 * (vb & 1) : 160 + 16 * (n - 8) + 2 * vb;
              const int grp = (sub * 32 + j) >> 3;
              const int k = j & 7;
              if (k < b) trec[grp * 288 + off + k] = uint8_t(w >> (8 * k));
            } else if (SYM4) {
              // packed and transposed after the block
            } else if (UB == 1) {
              // col layout, 1 bit: ballot over lanes = vectors; lanes 0..31
              // carry dim 32mb + r, lanes 32..63 dim 32mb + 16 + r
              const uint64_t m = __ballot((idx & 1) != 0);
              cw[nb][0] = (lane == r ? uint32_t(m) : cw[nb][0]);
              cw[nb][0] = (lane == 16 + r ? uint32_t(m >> 32) : cw[nb][0]);
            } else {
              // col layout, UB bits: the 32/UB vectors of a dword are OR-ed
              // together across their lanes (DPP butterfly); lane j of the
              // group keeps the dword of register r with r % VPD == j % VPD,
              // stored after the block.
              constexpr int VPD = 32 / UB;
              const uint32_t w = group_or<VPD>(uint32_t(idx) << (UB * (j & (VPD - 1))));
              if ((r % VPD) == (j & (VPD - 1))) colkeep[nb][r / VPD] = w;
            }
            if (MODE == 1 && SPLIT) {
              const bool og = SPLIT == 1 ? (r < 8 && !hh) : (16 * hh + r < cv.o4);
              const float rsd = fmaf(v, og ? rso[nb] : rsr[nb], -chat);  // 32 (y - c), own group's unit
              if (SPLIT == 2 || r < 8) {
                rro[nb] = fmaf(rsd, og ? rsd : 0.f, rro[nb]);
                rr[nb] = fmaf(rsd, og ? 0.f : rsd, rr[nb]);
              } else {
                rr[nb] = fmaf(rsd, rsd, rr[nb]);
              }
              acc[nb][r] = rsd;
            } else if (MODE == 1) {
              const float rsd = fmaf(v, rs[nb], -chat);  // 32 (y - c) in unit scale
              rr[nb] = fmaf(rsd, rsd, rr[nb]);
              acc[nb][r] = rsd;
            } else if (MODE == 2) {
              const float res = v - chat;
              if (mb == 0 && hh == 0 && r < 4) {
                rsmall[nb][r] = dim < cv.m ? res : 0.f;
                if (dim < cv.m) rr[nb] = fmaf(res, res, rr[nb]);
              }
            }
          }
          if constexpr (SYM2) sym2_finish(cw[nb][0], cw[nb][NPL - 1], 0xffffu);
          if constexpr (SPLIT == 1) cw[nb][0] ^= 0xffffu;  // complemented pushes
          if constexpr (SPLIT == 2) cw[nb][0] = gw[nb][0];  // plane 0: every coordinate
          if (!COL) {
            // row layout: half hh holds bits 16 hh .. 16 hh + 15 of each word;
            // slots past the end of the input are zero
            const int slot = sub * 32 * NB + nb * 32 + j;
#pragma unroll
            for (int p = 0; p < NPL; ++p) {
              const uint32_t mine = valid[nb] ? cw[nb][p] << (16 * hh) : 0u;
              const uint32_t w = mine | xor32(mine);
              // both halves hold the same word: an unconditional store keeps
              // the number of memory operations the same on every path
              *reinterpret_cast<uint32_t*>(trec + size_t(p) * kTile * 16 + slot * 16 + 4 * mb) = w;
            }
            if constexpr (SPLIT == 2) {
              // planes 1..: plane p holds the coordinates with more than p
              // index bits in stored order (both groups, or one), so block
              // mb's bits are one run of n_p in {32, o4, 32 - o4} bits at
              // base_p + n_p mb, byte-aligned; the bit string is stored in
              // 16-byte chunks of 64 vectors (a shorter last chunk)
              const int o4 = cv.o4;
              int base = 4 * 32;
              for (int p = 1; p < kMaxBits; ++p) {
                const bool co = p < cv.split_ub_o, cr = p < cv.split_ub_r;
                if (!co && !cr) break;
                const int np = (co ? o4 : 0) + (cr ? 32 - o4 : 0);
                const uint32_t mine = valid[nb] ? gw[nb][p] << (16 * hh) : 0u;
                uint32_t w = mine | xor32(mine);
                if (!co) w >>= o4;
                else if (!cr) w &= (1u << o4) - 1u;
                const int start = (base + np * mb) >> 3;  // first byte of the run
                if (hh == 0) {
                  for (int bt = 0; bt < np / 8; ++bt) {
                    const int B = start + bt, c = B >> 4;
                    const int wc = min(16, cv.code_bytes - 16 * c);
                    trec[size_t(c) * kTile * 16 + size_t(slot) * wc + (B & 15)] = uint8_t(w >> (8 * bt));
                  }
                }
                base += 4 * np;
              }
            }
          }
          if (SYM4) {
            // lane j holds the nibbles of registers 8k .. 8k + 7 of vector j;
            // after the 8-lane transposes lane j holds register
            // r = 8k + (j % 8) of vectors 8 (j / 8) .. 8 (j / 8) + 7, which is
            // the col dword of dim 32mb + 16hh + r for those vectors
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const uint32_t w = nib_transpose8(valid[nb] ? pk[nb][k] : 0u, nibc);
              const int r = 8 * k + (j & 7);
              const int dim = 32 * mb + 16 * hh + r;
              const int word = (sub * NB * 32 + nb * 32 + j) / 8;
              *reinterpret_cast<uint32_t*>(trec + size_t(dim) * 32 + 4 * word) = w;
            }
          }
          if (COL && UB > 1 && !SYM4 && !SPLIT) {
            // lane j holds, for r = k*VPD + (j % VPD), the dword of dim
            // 32mb + 16hh + r covering vectors (j / VPD)*VPD ..
            constexpr int VPD = 32 / UB;
#pragma unroll
            for (int k = 0; k < 16 / VPD; ++k) {
              const int r = k * VPD + (j & (VPD - 1));
              const int dim = 32 * mb + 16 * hh + r;
              const int word = (sub * NB * 32 + nb * 32 + j) / VPD;
              *reinterpret_cast<uint32_t*>(trec + size_t(dim) * 8 * UB + 4 * word) = colkeep[nb][k];
            }
          }
          if (COL && UB == 1 && !SPLIT) {
            // store the 32 dims x 32 vectors of this block: lane k < 32 holds dim 32mb+k
            if (lane < 32) {
              uint8_t* w = trec + (size_t(32) * mb + lane) * 8;
              const int half = sub * NB + nb;  // which 32-vector half of the 64-bit word
              *reinterpret_cast<uint32_t*>(w + 4 * half) = cw[nb][0];
            }
          }
        }
        // ------------------------------------------------ sketch block
        if (MODE == 1) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            u32x4 rh[NB], rl[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              float v[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) v[i] = acc[nb][8 * q + i];
              split8h(v, rh[nb], rl[nb], m1);
            }
            const int chunk = 2 * mb + q;
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
              const int off = (32 * ms + j) * LDS_ROW + 16 * chunk + 8 * hh;
              const u32x4 sh = *reinterpret_cast<const u32x4*>(sSk + off);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) {
                z[nb][ms] = mfma32h(sh, rh[nb], z[nb][ms]);
                z[nb][ms] = mfma32h(sh, rl[nb], z[nb][ms]);
              }
            }
          }
        }
      };
      if constexpr (PIPE) {
        // software pipeline: the rotation MFMAs of block mb + 1 are issued
        // ahead of the quantization of block mb, which does not depend on
        // them, so the matrix cores and the vector ALU work at the same time
        f32x16 a0[NB], a1[NB];
        rotate(0, a0);
        rotate(1, a1);
        block(0, a0);
        rotate(2, a0);
        block(1, a1);
        rotate(3, a1);
        block(2, a0);
        block(3, a1);
      } else {
#pragma unroll 1
        for (int mb = 0; mb < 4; ++mb) {
          f32x16 acc[NB];
          rotate(mb, acc);
          block(mb, acc);
        }
      }

      // ---------------------------------------------------- signs, norms
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int slot = sub * 32 * NB + nb * 32 + j;
        if (MODE == 1) {
          rr[nb] += xor32f(rr[nb]);
          if (SPLIT) rro[nb] += xor32f(rro[nb]);
          // register r of half hh of block ms holds sketch row 32 ms + 16 hh + r
#pragma unroll
          for (int ms = 0; ms < 4; ++ms) {
            if (!COL) sw[nb][ms] = valid[nb] ? sign_word16(z[nb][ms]) : 0u;
          }
        } else if (MODE == 2) {
          if (hh == 0) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              if (jj < cv.m) {
                float zz = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (i < cv.m) zz = fmaf(cv.sketch[jj * cv.m + i], rsmall[nb][i], zz);
                zsmall[nb][jj] = zz;
                if (zz >= 0.f && valid[nb]) sw[nb][0] |= 1u << jj;
              }
            }
          }
        }
        // combine the two half-waves' bits (row layout)
        if (!COL) {
          if (!UNIFORM && !SPLIT) tailw[nb] |= xor32(tailw[nb]);
          if (MODE == 1) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t mine = sw[nb][q] << (16 * hh);
              sw[nb][q] = mine | xor32(mine);
            }
          }
          if constexpr (SPLIT == 1) {
            // plane 1 (4 bytes per vector, [64][4] at 64 * 16): bit 8 mb + r =
            // bit 1 of outlier coordinate 8 mb + r; block mb's pushes sit in
            // byte 3 - mb, hence the byte swap
            const uint32_t mine = hh ? 0u : __builtin_bswap32(~p1w[nb]);  // complemented pushes
            const uint32_t w = valid[nb] ? (mine | xor32(mine)) : 0u;
            *reinterpret_cast<uint32_t*>(trec + size_t(kTile) * 16 + size_t(slot) * 4) = w;
          } else if (!UNIFORM && !SPLIT) {
            const int tb = cv.code_bytes - 16;  // tail bytes per vector (1..4)
            for (int k = 0; k < tb; ++k)
              trec[size_t(kTile) * 16 + size_t(slot) * tb + k] = uint8_t(tailw[nb] >> (8 * k));
          }
          if (MODE == 1) {
            uint8_t* dst = trec + cv.off_signs + slot * 16 + 8 * hh;
            *reinterpret_cast<u32x2*>(dst) = hh ? u32x2{sw[nb][2], sw[nb][3]}
                                                : u32x2{sw[nb][0], sw[nb][1]};
          } else if (MODE == 2) {
            sw[nb][0] |= xor32(sw[nb][0]);  // only half 0 formed the small sketch
            for (int k = 0; k < cv.sign_bytes; ++k)
              trec[cv.off_signs + size_t(slot) * cv.sign_bytes + k] = uint8_t(sw[nb][0] >> (8 * k));
          }
        }
        // both halves store the same norms (no divergent branch around stores)
        if (MODE == 2) rr[nb] += xor32f(rr[nb]);  // only half 0 summed the small residual
        {
          const float nx = valid[nb] ? nxv[nb] : 0.f;
          *reinterpret_cast<uint16_t*>(trec + cv.off_nx + 2 * slot) = f16_bits(nx);
          if (MODE != 0) {
            // prod: rr sums (32 r)^2 in unit scale; SQ: r^2 in accumulator scale
            const float nr = !valid[nb] ? 0.f : (MODE == 1 ? sqrtf(rr[nb]) * (1.f / 32.f) : sqrtf(rr[nb]) / wsc[nb]);
            *reinterpret_cast<uint16_t*>(trec + cv.off_nr + 2 * slot) = f16_bits(nr);
          }
          if constexpr (SPLIT) {  // the outlier instance's norms
            *reinterpret_cast<uint16_t*>(trec + cv.off_nxo + 2 * slot) = f16_bits(valid[nb] ? nxo[nb] : 0.f);
            if (MODE == 1)
              *reinterpret_cast<uint16_t*>(trec + cv.off_nro + 2 * slot) =
                  f16_bits(valid[nb] ? sqrtf(rro[nb]) * (1.f / 32.f) : 0.f);
          }
        }
      }
    }
  };
  // Jobs of this workgroup: job j is tile (j / nwaves) tstep + bx
  // nwaves + j % nwaves (both of its sub-tiles when NSUB = 2, else one
  // sub-tile).  Wave w starts with job w.  When the workgroup has at least
  // 4 jobs per wave, each further job goes to the wave that asks first (a
  // counter in LDS): the two waves sharing a SIMD are not issued at equal
  // rates, and a fixed split leaves the slower one last.  With fewer, a
  // late extra job costs more than the imbalance, and wave w keeps jobs
  // w, w + nwaves, ...
  __shared__ int sJob;
  const bool dyn = ntiles >= 4 * tstep;
  auto next_tile = [&](int64_t tl) {
    if (!dyn) return tl + tstep;  // uniform over the workgroup
    const int jb = take_job(&sJob, lane);
    const int r = jb / nwaves;
    return int64_t(r) * tstep + int64_t(bx) * nwaves + (jb - r * nwaves);
  };
  int64_t tile = int64_t(bx) * nwaves + wave;
  if (threadIdx.x == 0) sJob = nwaves;
  // the tables' loads go out first, then the first rows; the tables are
  // stored to LDS as soon as they arrive, with the rows still in flight
  {
    constexpr int NM = MODE == 1 ? 3 : 2;  // Pi hi, Pi lo (, S)
    const uint16_t* src[NM];
    uint16_t* dst[NM];
    bool perm[NM];
    src[0] = cv.rot_hi + size_t(hc) * D * D, dst[0] = sPiHi, perm[0] = false;
    src[1] = cv.rot_lo + size_t(hc) * D * D, dst[1] = sPiLo, perm[1] = false;
    if constexpr (NM == 3) src[2] = cv.sk_hi, dst[2] = sSk, perm[2] = true;
    u32x4 sv[NM][kStagePer];
    stage_load<NM>(src, sv);
    __builtin_amdgcn_sched_barrier(0);  // keep the two groups of loads in this order
    if (BF16IN) load_raw(tile, 0, bufA);
    __builtin_amdgcn_sched_barrier(0);
    stage_store<NM>(dst, perm, sv);
  }
  if constexpr (SYM4) {
    // bucket table of the 15 boundaries: entry e = (position of the
    // boundary inside bucket e, or +inf; number of boundaries below it),
    // positions y qinvw + qoff in bucket units
    for (int e = threadIdx.x; e < cv.qn; e += blockDim.x) {
      float thr = INFINITY;
      int below = 0;
#pragma unroll
      for (int k = 0; k < 15; ++k) {
        const float pos = fmaf(cv.uthr[k], cv.qinvw, cv.qoff);
        if (pos < float(e)) ++below;
        else if (pos < float(e + 1)) thr = pos;
      }
      sQ[e] = float2{thr, __int_as_float(below)};
    }
  }
  if (!UNIFORM && SPLIT != 1) {
    for (int e = threadIdx.x; e < D * kMaxLevels; e += blockDim.x) {
      sThr[e] = cv.thr[size_t(hc) * D * kMaxLevels + e];
      sCen[e] = cv.cen[size_t(hc) * D * kMaxLevels + e];
    }
  }
  __syncthreads();
  if constexpr (NB == 1) {
    // one tile per job: its second half is loaded while the first is
    // processed, the next job's first half while the second is
    while (tile < ntiles) {
      if (BF16IN) load_raw(tile, 1, bufB);
      process(bufA, tile, 0);
      const int64_t t1 = next_tile(tile);
      if (BF16IN) load_raw(t1, 0, bufA);
      process(bufB, tile, 1);
      tile = t1;
    }
  } else {
    // two 32-vector blocks per sub-tile: one code path, the prefetched set
    // is copied (two alternating instances would not fit the registers)
    while (tile < ntiles) {
      const int64_t t1 = next_tile(tile);
      if (BF16IN) load_raw(t1, 0, bufB);
      process(bufA, tile, 0);
      if (BF16IN) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int c = 0; c < 8; ++c) bufA[nb][c] = bufB[nb][c];
      }
      tile = t1;
    }
  }
}

// One codec: gx workgroups per (sequence, head) set along grid x; the sets
// run along grid y, continued in grid z past 65535.
template <int NB, bool BF16IN, int MODE, bool COL, bool UNIFORM, int UB, int SPLIT = 0>
__global__ __launch_bounds__(512, 1) void encode_d128_kernel(CodecView cv, EncodeArgs a) {
  encode_d128_body<NB, BF16IN, MODE, COL, UNIFORM, UB, SPLIT>(cv, a, int(blockIdx.x), int(gridDim.x),
                                                              blockIdx.y + int64_t(blockIdx.z) * gridDim.y);
}

// Keys and values of the same tokens in one launch (bf16 rows, uniform
// codecs): a 1-D grid whose first nk = kgx x (key sets) workgroups encode the
// keys and the rest the values.  Workgroups start in grid order, one per CU
// (the LDS tables), so the value workgroups fill the CUs the key workgroups
// leave, instead of waiting for the last of them as a second launch would.
template <int KMODE, int KUB, int VMODE, bool VCOL, int VUB>
__global__ __launch_bounds__(512, 1) void encode_kv_d128_kernel(CodecView kcv, EncodeArgs ka, int kgx,
                                                                CodecView vcv, EncodeArgs va, int vgx) {
  const int64_t nk = int64_t(kgx) * ka.batch * ka.heads;
  const int64_t wg = blockIdx.x;
  if (wg < nk)
    encode_d128_body<1, true, KMODE, false, true, KUB>(kcv, ka, int(wg % kgx), kgx, wg / kgx);
  else
    encode_d128_body<1, true, VMODE, VCOL, true, VUB>(vcv, va, int((wg - nk) % vgx), vgx, (wg - nk) / vgx);
}

// ---------------------------------------------------------------------------
// Randomized Hadamard rotation (Pi = H diag(s) / sqrt(d)), bf16 input, uniform
// codebooks.  The rotation is a fast Walsh-Hadamard transform in registers
// instead of the two MFMA passes of a dense Pi; the QJL sketch stays on MFMA.
//
// Lane (j, hh) holds input dims 64 hh .. 64 hh + 63 of vector j.  After the
// sign flips (XOR of the bf16 sign bits) and six in-lane butterfly stages,
// element t holds u_t of its half; the last stage pairs the two halves: a
// permlane32 swap of registers t and t + 32 leaves, in lane half hh,
// P_t = y_{32 hh + t} and M_t = y_{64 + 32 hh + t} (t < 32, y = H s x
// unnormalised).  So each lane owns two whole 32-dim blocks (mb = hh and
// mb = 2 + hh): its ROW words need no cross-half merge, and for the sketch
// the K order (chunk c, half hh, element i) -> dim of register 8c + i is
// matched by permuting the columns of S when it is staged.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int had_dim(int hh, int k) {  // dim held in register k (0..63) of half hh
  return k < 32 ? 32 * hh + k : 64 + 32 * hh + (k - 32);
}
static_assert(had_dim(0, 0) == 0 && had_dim(1, 0) == 32 && had_dim(0, 32) == 64 && had_dim(1, 63) == 127,
              "the two halves' registers cover dims 0..127 in blocks of 32");

// Stage S (fp16 [128][128]) with rows placed by lds_row_of and LDS column
// 16c + 8h + i holding S column had_dim(h, 8c + i).
__device__ void stage_sketch_had(uint16_t* lds, const uint16_t* g) {
  constexpr int CHUNKS = D * D / 8;
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int base = 0; base < CHUNKS; base += 8 * nt) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = base + u * nt + tid;
      if (e < CHUNKS) v[u] = *reinterpret_cast<const u32x4*>(g + e * 8);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = base + u * nt + tid;
      if (e >= CHUNKS) continue;
      const int row = e / (D / 8), col = (e % (D / 8)) * 8;  // 8 consecutive S columns
      // col = had_dim(h, 8c): dims 0..31 -> h 0, c 0..3; 32..63 -> h 1, c 0..3;
      // 64..95 -> h 0, c 4..7; 96..127 -> h 1, c 4..7
      const int h = (col >> 5) & 1, c = (col & 31) / 8 + 4 * (col >> 6);
      *reinterpret_cast<u32x4*>(lds + lds_row_of(row) * LDS_ROW + 16 * c + 8 * h) = v[u];
    }
  }
}

template <int MODE, bool COL, int UB>
__global__ __launch_bounds__(512, 1) void encode_had_kernel(CodecView cv, EncodeArgs a) {
  // MODE 0: mse (COL with 4 index bits, or ROW); MODE 1: prod with the full
  // 128-dim sketch (ROW)
  static_assert(MODE == 0 || !COL, "prod records are ROW");
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* sMask = reinterpret_cast<uint32_t*>(smem);           // [2][32] sign-bit masks
  uint16_t* sSk = reinterpret_cast<uint16_t*>(smem + 256);        // MODE 1: staged S
  const int64_t bh = blockIdx.y + int64_t(blockIdx.z) * gridDim.y;
  if (bh >= a.batch * a.heads) return;
  const int64_t b = bh / a.heads, h = bh % a.heads;
  // COL: bucket table of the 15 boundaries (one compare per coordinate, as
  // in the dense-rotation kernel)
  __shared__ float2 sQ[COL ? kQMax : 1];
  if (threadIdx.x < 64) sMask[threadIdx.x] = cv.had_mask[threadIdx.x];
  if (MODE == 1) stage_sketch_had(sSk, cv.sk_hi);
  if constexpr (COL) {
    for (int e = threadIdx.x; e < cv.qn; e += blockDim.x) {
      float thr = INFINITY;
      int below = 0;
#pragma unroll
      for (int k = 0; k < 15; ++k) {
        const float pos = fmaf(cv.uthr[k], cv.qinvw, cv.qoff);
        if (pos < float(e)) ++below;
        else if (pos < float(e + 1)) thr = pos;
      }
      sQ[e] = float2{thr, __int_as_float(below)};
    }
  }
  __syncthreads();

  const int lane = lane_id();
  const int j = lane & 31, hh = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int64_t ntiles = (a.tokens + kTile - 1) / kTile;
  const uint8_t* xbase = static_cast<const uint8_t*>(a.x) + (b * a.xs_b + h * a.xs_h) * 2;
  uint8_t* rbase = a.rec + b * a.rs_b + h * a.rs_h;
  constexpr int LV = 1 << UB;
  constexpr bool SYM4 = COL && UB == 4;
  constexpr bool SYM2 = !COL && UB == 2;
  static_assert(!COL || SYM4, "col records: 4 index bits");
  const NibT nibc = nib_transpose_consts(int(threadIdx.x & 7));
  const float kSqrtD = 11.313708498984761f;  // sqrt(128): y = FWHT / sqrt(d)

  const int nwaves = blockDim.x >> 6;
  const int64_t tstep = int64_t(gridDim.x) * nwaves;
  u32x4 bufA[8], bufB[8];
  auto load_raw = [&](int64_t tl, int sb, u32x4 (&dst)[8]) {
    const int64_t t = tl * kTile + sb * 32 + j;
    const int64_t tc = (tl < ntiles && t < a.tokens) ? t : a.tokens - 1;
    const uint16_t* row = reinterpret_cast<const uint16_t*>(xbase) + tc * a.xs_t + 64 * hh;
#pragma unroll
    for (int c = 0; c < 8; ++c) dst[c] = *reinterpret_cast<const u32x4*>(row + 8 * c);
  };
  auto process = [&](const u32x4 (&cur)[8], int64_t tile, int sub) {
    uint8_t* trec = rbase + tile * cv.tile_bytes;
    const float m1 = opaque_minus_one();
    const int slot = sub * 32 + j;
    const bool valid = tile * kTile + slot < a.tokens;
    // ------------------------------------------------ signs, norm, unpack
    float v[64];
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 m = *reinterpret_cast<const u32x4*>(sMask + 32 * hh + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = cur[c][i] ^ m[i];
        const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
        v[8 * c + 2 * i] = lo;
        v[8 * c + 2 * i + 1] = hi;
        s0 = fmaf(lo, lo, s0);
        s1 = fmaf(hi, hi, s1);
      }
    }
    float ss = s0 + s1;
    ss += xor32f(ss);
    // ------------------------------------------------ Walsh-Hadamard
#pragma unroll
    for (int st = 1; st < 64; st <<= 1)
#pragma unroll
      for (int t = 0; t < 64; ++t)
        if (!(t & st)) {
          const float p = v[t], q = v[t + st];
          v[t] = p + q;
          v[t + st] = p - q;
        }
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[t]), __float_as_uint(v[t + 32]), false, false);
      const float A = __uint_as_float(sw[0]), B = __uint_as_float(sw[1]);
      v[t] = A + B;       // P_t: dim 32 hh + t
      v[t + 32] = A - B;  // M_t: dim 64 + 32 hh + t
    }
    // Norms below 2^-50 (whose squares may be denormal or flushed) and zero
    // vectors: the wave scales every transformed vector by 2^e from its
    // largest coordinate and sums the squares again (the transform has
    // sum (Hx)_i^2 = 128 ||x||^2).  The scaling is exact and commutes with
    // the butterflies, so vectors of ordinary size get the same values as
    // without it.  Zeros become +0 here: the sign flips make -0 inputs and a
    // butterfly of two -0 is -0, which only an all-zero vector can carry to
    // the output, where the quantizer reads sign bits.  Placed after the
    // transform, so that the butterflies overlap the norm's reduction.
    float nd = 1.f;  // stored norm = sqrt(ss) / nd
    if (__ballot(!(ss >= 0x1p-100f)) != 0) {
      float mx = 0.f;
#pragma unroll
      for (int t = 0; t < 64; ++t) mx = fmaxf(mx, fabsf(v[t]));
      mx = fmaxf(mx, xor32f(mx));
      const int ebits = int((__float_as_uint(mx) >> 23) & 0xff);
      nd = mx > 0.f ? __uint_as_float(uint32_t(min(254, max(1, 268 - ebits))) << 23) : 1.f;
      float q0 = 0.f, q1 = 0.f;
#pragma unroll
      for (int t = 0; t < 64; t += 2) {
        v[t] = v[t] * nd + 0.f;  // -0 -> +0
        v[t + 1] = v[t + 1] * nd + 0.f;
        q0 = fmaf(v[t], v[t], q0);
        q1 = fmaf(v[t + 1], v[t + 1], q1);
      }
      ss = q0 + q1;
      ss += xor32f(ss);
      ss *= 1.f / 128.f;
    }
    const float nxv = sqrtf(ss) / nd;
    const float sx = ss > 0.f ? sqrtf(ss) : 1.f;  // a zero vector encodes y = 0
    const float wsc = kSqrtD * sx;                // accumulator = wsc * (unit-vector coordinate)
    // ------------------------------------------------ quantize
    f32x16v T = {};
#pragma unroll
    for (int k = 0; k < LV - 1; ++k) T[k] = cv.uthr[k] * wsc;
    const float sK = SYM4 ? cv.qinvw / wsc : 0.f;  // bucket units per accumulator unit
    float C32[LV];
#pragma unroll
    for (int k = 0; k < LV; ++k) C32[k] = 32.f * cv.ucen[k];
    const float rs = 32.f / wsc;
    float rr = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {  // dims 32 mb .. 32 mb + 31, mb = hh + 2 blk
      const int mb = hh + 2 * blk;
      if constexpr (COL) {
        // nibbles of 8 consecutive dims per word, then the 8-lane transpose
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t w = 0;
#pragma unroll
          for (int i = 7; i >= 0; --i) {
            const float u = __builtin_amdgcn_fmed3f(fmaf(v[32 * blk + 8 * g + i], sK, cv.qoff), 0.f,
                                                    float(cv.qn - 1));
            const float2 e = sQ[uint32_t(u)];
            w = (w << 4) + uint32_t(__float_as_int(e.y)) + (u >= e.x ? 1u : 0u);
          }
          w = nib_transpose8(valid ? w : 0u, nibc);
          const int dim = 32 * mb + 8 * g + (j & 7);
          *reinterpret_cast<uint32_t*>(trec + size_t(dim) * 32 + 4 * (slot / 8)) = w;
        }
      } else {
        uint32_t cw[UB];
#pragma unroll
        for (int p = 0; p < UB; ++p) cw[p] = 0;
#pragma unroll
        for (int r = 31; r >= 0; --r) {  // descending: dim 32 mb + r lands at bit r
          const float val = v[32 * blk + r];
          float chat;
          if constexpr (SYM2) {
            chat = quant2_sym_push(val, T[2], C32[2], C32[3], cw[0], cw[1]);
          } else {
            bool bits[4] = {false, false, false, false};
            chat = quant_bits<UB>(val, T, C32, bits);
#pragma unroll
            for (int p = 0; p < UB; ++p) cw[p] = push_bit(cw[p], bits[p]);
          }
          if (MODE == 1) {
            const float rsd = fmaf(val, rs, -chat);  // 32 (y - c) in unit scale
            rr = fmaf(rsd, rsd, rr);
            v[32 * blk + r] = rsd;
          }
        }
        if constexpr (SYM2) sym2_finish(cw[0], cw[1], 0xffffffffu);
#pragma unroll
        for (int p = 0; p < UB; ++p)
          *reinterpret_cast<uint32_t*>(trec + size_t(p) * kTile * 16 + slot * 16 + 4 * mb) = valid ? cw[p] : 0u;
      }
    }
    // ------------------------------------------------ sketch and signs
    if constexpr (MODE == 1) {
      f32x16 z[4];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4 rh, rl;
        split8h(&v[8 * c], rh, rl, m1);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          const u32x4 sh = *reinterpret_cast<const u32x4*>(sSk + (32 * ms + j) * LDS_ROW + 16 * c + 8 * hh);
          z[ms] = mfma32h(sh, rh, c == 0 ? f32x16{} : z[ms]);
          z[ms] = mfma32h(sh, rl, z[ms]);
        }
      }
      rr += xor32f(rr);
      uint32_t sw[4];
      // register r of half hh of block ms holds sketch row 32 ms + 16 hh + r
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const uint32_t mine = valid ? sign_word16(z[ms]) << (16 * hh) : 0u;
        sw[ms] = mine | xor32(mine);
      }
      uint8_t* dst = trec + cv.off_signs + slot * 16 + 8 * hh;
      *reinterpret_cast<u32x2*>(dst) = hh ? u32x2{sw[2], sw[3]} : u32x2{sw[0], sw[1]};
    }
    // ------------------------------------------------ norms (both halves store the same)
    *reinterpret_cast<uint16_t*>(trec + cv.off_nx + 2 * slot) = f16_bits(valid ? nxv : 0.f);
    if (MODE == 1)
      *reinterpret_cast<uint16_t*>(trec + cv.off_nr + 2 * slot) =
          f16_bits(valid ? sqrtf(rr) * (1.f / 32.f) : 0.f);
  };
  // jobs handed out as in encode_d128_kernel (one tile, both sub-tiles, per
  // job; from the counter with at least 4 jobs per wave); the counter
  // starts once the barrier below has passed
  __shared__ int sJob;
  const bool dyn = ntiles >= 4 * tstep;
  auto next_tile = [&](int64_t tl) {
    if (!dyn) return tl + tstep;  // uniform over the workgroup
    const int jb = take_job(&sJob, lane);
    const int r = jb / nwaves;
    return int64_t(r) * tstep + int64_t(blockIdx.x) * nwaves + (jb - r * nwaves);
  };
  int64_t tile = int64_t(blockIdx.x) * nwaves + wave;
  if (threadIdx.x == 0) sJob = nwaves;
  __syncthreads();
  load_raw(tile, 0, bufA);
  while (tile < ntiles) {
    load_raw(tile, 1, bufB);
    process(bufA, tile, 0);
    const int64_t t1 = next_tile(tile);
    load_raw(t1, 0, bufA);
    process(bufB, tile, 1);
    tile = t1;
  }
}

// Grid of gx workgroups per (sequence, head) set: the sets run along y and,
// past 65535, along z (the kernels skip the padding of the last z plane).
dim3 set_grid(int64_t gx, int64_t sets) {
  const int64_t sy = std::min<int64_t>(sets, 65535);
  return dim3(unsigned(gx), unsigned(sy), unsigned((sets + sy - 1) / sy));
}

template <int MODE, bool COL, int UB>
hipError_t launch_had(const CodecView& cv, const EncodeArgs& a, hipStream_t s) {
  auto kern = encode_had_kernel<MODE, COL, UB>;
  const size_t lds = 256 + (MODE == 1 ? size_t(D) * LDS_ROW * 2 : 0);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const int64_t ntiles = (a.tokens + kTile - 1) / kTile;
  const int64_t sets = a.batch * a.heads;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  int64_t gx = (ntiles + 7) / 8;
  const int64_t want = std::max<int64_t>(1, (int64_t(cus) + sets - 1) / sets);
  gx = std::max<int64_t>(1, std::min(gx, want));
  hipLaunchKernelGGL(kern, set_grid(gx, sets), dim3(512), lds, s, cv, a);
  return hipGetLastError();
}

// Dynamic LDS of the d = 128 encode: Pi hi and lo, S for a full sketch, the
// per-dim tables of non-uniform codecs.
template <int MODE, bool UNIFORM, int SPLIT>
constexpr size_t encode_lds() {
  return size_t(2) * D * LDS_ROW * 2 + (MODE == 1 ? size_t(D) * LDS_ROW * 2 : 0) +
         (!UNIFORM && SPLIT != 1 ? size_t(2) * D * kMaxLevels * 4 : 0);
}

// Workgroups per (sequence, head) set: one 8-wave workgroup per CU (the LDS
// copy of Pi/S) each looping over tiles, as many as the sets leave CUs for,
// and at least 8 tiles each.
int64_t encode_gx(const EncodeArgs& a) {
  const int64_t ntiles = (a.tokens + kTile - 1) / kTile;
  const int64_t sets = a.batch * a.heads;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int64_t gx = (ntiles + 7) / 8;
  const int64_t want = std::max<int64_t>(1, (int64_t(cus) + sets - 1) / sets);
  return std::max<int64_t>(1, std::min(gx, want));
}

template <int NB, bool BF16IN, int MODE, bool COL, bool UNIFORM, int UB, int SPLIT = 0>
hipError_t launch_one(const CodecView& cv, const EncodeArgs& a, hipStream_t s) {
  auto kern = encode_d128_kernel<NB, BF16IN, MODE, COL, UNIFORM, UB, SPLIT>;
  const size_t lds = encode_lds<MODE, UNIFORM, SPLIT>();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, set_grid(encode_gx(a), a.batch * a.heads), dim3(512), lds, s, cv, a);
  return hipGetLastError();
}

template <int KMODE, int KUB, int VMODE, bool VCOL, int VUB>
hipError_t launch_kv(const CodecView& kcv, const EncodeArgs& ka, const CodecView& vcv, const EncodeArgs& va,
                     hipStream_t s) {
  auto kern = encode_kv_d128_kernel<KMODE, KUB, VMODE, VCOL, VUB>;
  const size_t lds = std::max(encode_lds<KMODE, true, 0>(), encode_lds<VMODE, true, 0>());
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const int64_t kgx = encode_gx(ka), vgx = encode_gx(va);
  const int64_t wgs = (kgx + vgx) * ka.batch * ka.heads;
  if (wgs > INT32_MAX) return hipErrorNotSupported;
  hipLaunchKernelGGL(kern, dim3(unsigned(wgs)), dim3(512), lds, s, kcv, ka, int(kgx), vcv, va, int(vgx));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_encode_kv_d128(const CodecView& kcv, const EncodeArgs& ka, const CodecView& vcv,
                                 const EncodeArgs& va, hipStream_t s) {
  // one launch for the prod b = 3 ROW keys and mse b = 4 COL values of bf16
  // rows with a dense Pi (the KV-cache pair the pages quantize); any other
  // pair as the two launches of launch_encode_d128
  const bool pair = ka.x_bf16 && va.x_bf16 && ka.batch == va.batch && ka.heads == va.heads &&
                    ka.tokens == va.tokens && kcv.uniform && vcv.uniform && !kcv.had_mask && !vcv.had_mask &&
                    !kcv.outl && !vcv.outl && kcv.mode == TQ_PROD && kcv.m == D &&
                    kcv.layout == TQ_LAYOUT_ROW && kcv.ubits == 2 && vcv.mode == TQ_MSE &&
                    vcv.layout == TQ_LAYOUT_COL && vcv.ubits == 4 && vcv.qn >= 2 && vcv.qn <= kQMax;
  if (pair) {
    const hipError_t e = launch_kv<1, 2, 0, true, 4>(kcv, ka, vcv, va, s);
    if (e != hipErrorNotSupported) return e;
  }
  const hipError_t e = launch_encode_d128(kcv, ka, s);
  if (e != hipSuccess) return e;
  return launch_encode_d128(vcv, va, s);
}

hipError_t launch_encode_d128(const CodecView& cv, const EncodeArgs& a, hipStream_t s) {
  const bool col = cv.layout == TQ_LAYOUT_COL;
  if (cv.had_mask && cv.uniform && a.x_bf16) {
    // randomized Hadamard rotation: the register transform for the GQA K/V
    // codecs; any other combination uses the dense Pi below
    if (cv.mode == TQ_MSE && col && cv.ubits == 4 && cv.qn >= 2 && cv.qn <= kQMax)
      return launch_had<0, true, 4>(cv, a, s);
    if (cv.mode == TQ_PROD && !col && cv.m == D && cv.ubits == 2) return launch_had<1, false, 2>(cv, a, s);
  }
  if (cv.outl) {
    // outlier-channel split, row layout, full block sketch: the 2.5-bit KV
    // setting (32 outlier coordinates at 2 index bits, the others at 1) on
    // its specialised path, any other outlier count and bits on the general
    // one; col layout: 2.5-bit mse values (32 outlier coordinates at 3 index
    // bits, the others at 2) on the general path
    if (!cv.omask) return hipErrorNotSupported;
    if (col) {
      if (cv.mode != TQ_MSE || cv.o4 != 8 || cv.split_ub_o != 3 || cv.split_ub_r != 2) return hipErrorNotSupported;
      return a.x_bf16 ? launch_one<1, true, 0, true, false, 1, 2>(cv, a, s)
                      : launch_one<1, false, 0, true, false, 1, 2>(cv, a, s);
    }
    const bool fast = cv.o4 == 8 && cv.split_ub_o == 2 && cv.split_ub_r == 1;
    if (cv.mode == TQ_PROD) {
      if (cv.m != D) return hipErrorNotSupported;
      if (fast)
        return a.x_bf16 ? launch_one<1, true, 1, false, false, 1, 1>(cv, a, s)
                        : launch_one<1, false, 1, false, false, 1, 1>(cv, a, s);
      return a.x_bf16 ? launch_one<1, true, 1, false, false, 1, 2>(cv, a, s)
                      : launch_one<1, false, 1, false, false, 1, 2>(cv, a, s);
    }
    if (fast)
      return a.x_bf16 ? launch_one<1, true, 0, false, false, 1, 1>(cv, a, s)
                      : launch_one<1, false, 0, false, false, 1, 1>(cv, a, s);
    return a.x_bf16 ? launch_one<1, true, 0, false, false, 1, 2>(cv, a, s)
                    : launch_one<1, false, 0, false, false, 1, 2>(cv, a, s);
  }
  if (!cv.uniform) {
    // SpectralQuant keys: row layout, small sketch
    if (col || cv.mode != TQ_PROD || cv.m > 4 || !a.x_bf16) return hipErrorNotSupported;
    // UB = 2: the SpectralQuant structure (multi-bit dims 0..3 only)
    if (cv.sq_ok) return launch_one<1, true, 2, false, false, 2>(cv, a, s);
    return launch_one<1, true, 2, false, false, 1>(cv, a, s);
  }
  const int mode = cv.mode == TQ_MSE ? 0 : (cv.m == D ? 1 : 2);
  if (mode == 2) return hipErrorNotSupported;
#define TQ_DISPATCH_UB(NB, BF, MODE, COL)                                   \
  switch (cv.ubits) {                                                       \
    case 1: return launch_one<NB, BF, MODE, COL, true, 1>(cv, a, s);        \
    case 2: return launch_one<NB, BF, MODE, COL, true, 2>(cv, a, s);        \
    case 3: return launch_one<NB, BF, MODE, COL, true, 3>(cv, a, s);        \
    case 4: return launch_one<NB, BF, MODE, COL, true, 4>(cv, a, s);        \
    default: return hipErrorNotSupported;                                   \
  }
  if (col && cv.ubits == 3) return hipErrorNotSupported;
  // 16-level col codes take the bucket-table quantizer
  if (col && cv.ubits == 4 && mode == 0 && (cv.qn < 2 || cv.qn > kQMax)) return hipErrorNotSupported;
  if (a.x_bf16) {
    // mse values take 32 vectors per wave step (about 190 VGPRs) rather than
    // 64 (256): twice the sub-tiles per wave for the row prefetch to overlap;
    // on 8 x 32768 bf16 values 44.9 -> 36.8 us (col, b = 4), 46.8 -> 42.7 us
    // (row, b = 4)
    if (mode == 0) { if (col) { TQ_DISPATCH_UB(1, true, 0, true) } else { TQ_DISPATCH_UB(1, true, 0, false) } }
    else { if (col) return hipErrorNotSupported; TQ_DISPATCH_UB(1, true, 1, false) }
  } else {
    if (mode == 0) { if (col) { TQ_DISPATCH_UB(1, false, 0, true) } else { TQ_DISPATCH_UB(1, false, 0, false) } }
    else { if (col) return hipErrorNotSupported; TQ_DISPATCH_UB(1, false, 1, false) }
  }
#undef TQ_DISPATCH_UB
}

}  // namespace tq
