// Launch interfaces of the HIP kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tq {

// Everything the kernels read of a codebook, by value.
struct CodecView {
  int d, mode, m, layout, uniform, ubits, heads;
  int code_bytes, sign_bytes, tile_bytes;
  int off_signs, off_nx, off_nr;
  int tail_bits;  // ROW, non-uniform: index bits beyond plane 0 (<= 32)
  // outlier-channel split (stored order): stored coordinate i belongs to the
  // outlier instance when i % 32 < o4; its norms sit at off_nxo / off_nro
  int outl, o4, off_nxo, off_nro;
  const uint32_t* omask;       // split: [H][4] outlier-channel bit masks (bit c = channel c)
  int split_ub_o, split_ub_r;  // index bits of the outlier / regular instance
  int sq_ok;      // non-uniform with 1 bit on dims 4.. and 1..5 bits on dims 0..3
  const float* rot;
  const float* rot_t;    // transpose of rot
  const uint16_t* rot_hi;
  const uint16_t* rot_lo;
  const float* sketch;
  const float* sketch_t; // transpose of sketch
  const uint16_t* sk_hi;
  const uint16_t* sk_lo;
  const float* thr;
  const float* cen;
  const int16_t* bitpos;
  const uint8_t* dim_bits;
  const uint32_t* sq_tail;  // non-uniform d = 128: tail byte -> packed index bits of dims 0..3
  const float* sq_gm;       // non-uniform d = 128: [H][2][d] half-difference and mean of levels 0, 1
  const uint32_t* had_mask; // randomized Hadamard, d = 128: [2][32] XOR masks of the bf16 sign bits
  const float* had_sign;    // randomized Hadamard, d = 128: the signs s [d] as +-1.0f
  // d a multiple of 128 other than 128, uniform codecs: the MFMA operand tiles
  // [d/128][d/32][hi, lo][128][32] of 16 Pi and [m/128][m/32][128][32] of S
  const uint16_t* rot_tiles;
  const uint16_t* sk_tiles;
  float uthr[kMaxLevels];
  float ucen[kMaxLevels];
  // uniform codecs: bucket table of the boundaries for a one-compare
  // quantizer.  A coordinate y of the unit vector falls in bucket
  // floor(y qinvw + qoff) of qn buckets of width 1 / qinvw; every bucket
  // holds at most one boundary, none within 2 % of a bucket edge (qn = 0:
  // no table)
  int qn;
  float qinvw, qoff;
};
constexpr int kQMax = 512;  // largest bucket table

CodecView make_view(const tq_codebook* cb);

// Calibration moments (SpectralQuant rotation) of heads x n vectors of d
// coordinates (d a multiple of 32), fp64: per head the column sums [d], the
// second moment [d][d] and the second moment of the normalised vectors
// [d][d]; rinv2 is scratch of heads * n doubles.
hipError_t launch_calib_moments(const void* x, int bf16, int heads, int64_t n, int d, double* rinv2,
                                double* mom_x, double* mom_u, double* sum_x, hipStream_t s);

struct EncodeArgs {
  const void* x;
  int x_bf16;
  int64_t batch, heads, tokens, xs_b, xs_h, xs_t;
  uint8_t* rec;
  int64_t rs_b, rs_h;
};

hipError_t launch_encode_d128(const CodecView& cv, const EncodeArgs& a, hipStream_t s);
// keys and values of the same tokens, in one launch where the pair allows it
hipError_t launch_encode_kv_d128(const CodecView& kcv, const EncodeArgs& ka, const CodecView& vcv,
                                 const EncodeArgs& va, hipStream_t s);

// One new vector per (sequence, head) written into slot positions[b] of the
// existing records (d = 128).
struct AppendArgs {
  const void* x;        // [B][H][d] rows with strides xs_b, xs_h (elements)
  int x_bf16;
  int B, H;
  int64_t xs_b, xs_h;
  uint8_t* rec;         // set (b, h) at rec + b * rs_b + h * rs_h
  int64_t rs_b, rs_h;
  const int32_t* positions;  // [B]
  int capacity;         // tokens the records hold
  // paged records (block_table non-NULL): tile t of set (b, h) is tile
  // t % 2^page_shift of page block_table[(b * H + h) * max_pages + (t >> page_shift)]
  // of the pool rec; rs_b and rs_h are then unused
  const int32_t* block_table;
  int page_shift, max_pages;
};
bool append_supported(const CodecView& cv);
hipError_t launch_append(const CodecView& cv, const AppendArgs& a, hipStream_t s);
// The key and the value of a decode step in one launch (same B and H).
hipError_t launch_append_pair(const CodecView& kc, const AppendArgs& ka, const CodecView& vc,
                              const AppendArgs& va, hipStream_t s);

// q' = Pi_h q and qs = S q'[0:m] for nq queries; head_of_query maps query ->
// rotation head (NULL: all head 0; else head = (query / group) % hkv ...).
struct QueryPrepArgs {
  const void* q;
  int q_bf16;
  int64_t nq;
  int q_per_head;   // queries sharing one codebook head, consecutive (GQA group); 0 = fixed head
  int hkv;          // number of KV heads in the cycle (for [B][Hq] layouts)
  int fixed_head;
  float* qr;        // [nq][d]
  float* qs;        // [nq][m]
};
hipError_t launch_query_prep(const CodecView& cv, const QueryPrepArgs& a, hipStream_t s);

hipError_t launch_score(const CodecView& cv, const float* qr, const float* qs, int64_t nq,
                        const uint8_t* rec, int64_t n, float* scores, hipStream_t s, int head = 0);

struct DecodeArgs {
  const float* qr;     // [B][Hq][d]   (prepared queries; the MFMA kernel forms its own)
  const float* qs;     // [B][Hq][mk]
  const void* q;       // [B][Hq][d] raw queries (fp32 or bf16), read by the MFMA kernel
  int q_bf16;
  int B, Hq, Hkv;
  const uint8_t* krec;
  const uint8_t* vrec;
  int64_t ks_seq, ks_head, vs_seq, vs_head;
  int max_tokens;
  const int32_t* seq_lens;
  float scale;
  int chunk_tiles;     // tiles per split
  int nsplit;
  int waves;           // MFMA kernel: waves per workgroup, 4 or 8 (8 only with nsplit > 1)
  int len_add;         // tokens attended = min(seq_lens[b] + len_add, max_tokens)
  // paged records (block_table non-NULL): tile t of set (b, g) is tile
  // t % 2^page_shift of page block_table[(b * Hkv + g) * max_pages + (t >> page_shift)]
  // of the pools krec / vrec; the strides are then unused
  const int32_t* block_table;
  int page_shift, max_pages;
  float* part;         // workspace partials
  float* out;          // [B][Hq][d]
};

// Index, within its page pool, of tile t of set `row` (= b * H + h) of a
// paged cache: the page's first tile plus the tile's place in the page.
__device__ __forceinline__ int64_t paged_tile(const int32_t* block_table, int page_shift, int max_pages,
                                              int64_t row, int t) {
  const int pg = block_table[row * max_pages + (t >> page_shift)];
  return (int64_t(pg) << page_shift) + (t & ((1 << page_shift) - 1));
}
// Unnormalised Walsh-Hadamard transform in Sylvester order, y = H x with
// H[i][j] = (-1)^popcount(i & j), of a 128-vector held by one wave: lane l
// owns coordinates l (lo) and l + 64 (hi).  The stride-64 butterfly is within
// the lane, strides 32 .. 1 pair lane l with lane l ^ stride (the lower one
// keeps the sum, the upper one the difference).  The randomized Hadamard
// rotation Pi = H diag(s) / sqrt(d) is then Pi x = H (s x) / sqrt(d) and
// Pi^T y = s (H y) / sqrt(d), H being symmetric.
__device__ __forceinline__ void fwht128_wave(float& lo, float& hi, int lane) {
  const float a = lo + hi, b = lo - hi;
  lo = a;
  hi = b;
#pragma unroll
  for (int st = 32; st > 0; st >>= 1) {
    const float pl = __shfl_xor(lo, st, 64), ph = __shfl_xor(hi, st, 64);
    const bool up = (lane & st) != 0;
    lo = up ? pl - lo : lo + pl;
    hi = up ? ph - hi : hi + ph;
  }
}
constexpr float kInvSqrt128 = 0.08838834764831845f;  // 1 / sqrt(128)

hipError_t launch_decode(const CodecView& kv, const CodecView& vv, const DecodeArgs& a,
                         hipStream_t s);
// MFMA decode partial kernel (d = 128, prod keys with 1-2 index bits and a
// full sketch, mse values with 4 bits in col layout, 1-4 query heads per KV head).
bool decode_mfma_supported(const CodecView& kv, const CodecView& vv, int G);
hipError_t launch_decode_mfma(const CodecView& kv, const CodecView& vv, const DecodeArgs& a,
                              hipStream_t s);

// Per-query top-k of a [nq][cols] score block (row stride ld, ids id_base +
// column) into partial lists seg_base .. seg_base + nseg - 1 of total_seg.
// Scores are part[q][t] * row_scale[q] * col_scale[t] (each scale optional).
hipError_t launch_topk_segments(const float* scores, int64_t ld, int64_t cols, int64_t id_base,
                                int64_t nq, int k, int nseg, int seg_base, int total_seg,
                                float* ps, int64_t* pi, hipStream_t s,
                                const float* col_scale = nullptr, const float* row_scale = nullptr);
hipError_t launch_topk_merge(const float* ps, const int64_t* pi, int64_t nq, int total_seg, int k,
                             float* out_s, int64_t* out_i, hipStream_t s);

// Wide vectors (d a multiple of 128; encode and query preparation for d other
// than 128) and the MFMA search / dense scoring (tq_wide.hip).
int64_t wide_encode_chunk();
size_t wide_encode_workspace(const CodecView& cv);
hipError_t launch_encode_wide(const CodecView& cv, const EncodeArgs& a, void* ws, hipStream_t s);
size_t wide_query_prep_workspace(const CodecView& cv, int64_t nq);
hipError_t launch_query_prep_wide(const CodecView& cv, const float* q, int64_t nq, float* qr, float* qs,
                                  void* ws, hipStream_t s);
// Fused scoring + top-k (or dense scores) of uniform ROW codecs with 1..3
// index bits: 128 queries per workgroup, keys split over nsplit workgroups
// per query block, 4 partial lists (one per wave) per workgroup.
struct SearchPlan {
  int nqb, nsplit, nparts;
  int64_t keys_per_split;
  size_t tiles_bytes, inv_bytes;
};
bool search_mfma_supported(const CodecView& cv);
SearchPlan search_plan(const CodecView& cv, int64_t nq, int64_t n, int cus);
// dense != nullptr: scores [nq][n] are written instead of the top-k lists
hipError_t launch_search(const CodecView& cv, const float* qr, const float* qs, int64_t nq, const uint8_t* rec,
                         int64_t n, int k, const SearchPlan& p, void* tiles_ws, float* inv_ws, float* ps,
                         int64_t* pi, float* out_s, int64_t* out_i, float* dense, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

}  // namespace tq
