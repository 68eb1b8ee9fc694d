/*
 * tq.h -- C ABI of the TurboQuant / SpectralQuant codec for MI355X (gfx950).
 *
 * The library quantizes vectors online (TurboQuant: store ||x||, rotate
 * x/||x|| by a seeded random orthogonal Pi, quantize each rotated coordinate
 * with a precomputed Lloyd-Max codebook for the known post-rotation law; the
 * prod variant adds a 1-bit QJL sketch of the residual) and scores queries
 * directly against the compressed records (inner products, fused decode
 * attention, top-k search).
 *
 * Sources of the operations (web pages, cited by title and section):
 *   [TQ]  "TurboQuant: Online Vector Quantization with Near-optimal Distortion
 *         Rate" -- paper review (Zandieh et al., ICLR 2026): sections
 *         "Method", "Key idea", "Results", "Limitations", "Sparks".
 *   [SQ]  SpectralQuant thread (Ashwin Gopinath, tweet index), tweets 2-6.
 *   [LK]  OnlyTerp/turboquant LAUNCH.md (launch kit): dense-QR rotation mode.
 *
 * Conventions for every entry point:
 *   - All array arguments named as device buffers are device pointers on the
 *     codebook's device; host pointers are marked "host".
 *   - The caller owns every buffer.  Only tq_codebook_build allocates (device
 *     tables of the codebook) and tq_codebook_free releases them.
 *   - Argument, shape and alignment checks run before any launch; on error
 *     nothing is launched and nothing is written.  Kernel launches are
 *     asynchronous on `stream` (a hipStream_t, NULL = default stream); launch
 *     failures return TQ_EDEVICE, faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - Codebooks are immutable after build and may be shared across streams.
 *   - No function prints, throws or calls exit.
 *
 * Record layout (the pages define none; this is the library's own format).
 * Records are grouped in TILES of 64 consecutive vectors; a buffer holding n
 * records is ceil(n/64) tiles of tq_codebook_info.tile_bytes bytes.  Fields of
 * a tile, in order: codes, signs (prod only), n_x (64 x fp16), n_r (64 x fp16,
 * prod only); an outlier-split codec then adds the outlier instance's n_x and
 * (prod) n_r, and its n_x / n_r fields are the regular instance's.  Norms are
 * fp16, round to nearest even.
 *   ROW layout (for keys and database vectors, read one vector per lane):
 *     a vector's index bits form one bit string, plane by plane (plane p holds
 *     bit p of the index of every dim with more than p bits, dims ascending);
 *     bit k of the string is bit (k mod 8) of byte (k div 8).  Its
 *     C = ceil(B/8) bytes are cut into 16-byte chunks (the last may be
 *     shorter); chunk j of the tile is stored as [64 vectors][width_j] bytes.
 *     Sign bits (bit j = [z_j >= 0]) are packed and chunked the same way.
 *   COL layout (for values, read one coordinate per lane across the tile;
 *     uniform codecs only): for every dim i, ascending, a field of 8*b bytes
 *     holding the b-bit indices of the tile's 64 vectors, vector v at bits
 *     [b*v, b*v + b) (bit k of the field is bit k mod 8 of byte k div 8); then
 *     (prod) one little-endian 64-bit word per sketch dim j, bit v = sign bit
 *     of vector v.
 *   Slots past the last vector of a partly filled tile are written as zero.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = 1,        /* bad argument: null pointer, non-positive size, bad enum  */
  TQ_EUNSUPPORTED = 2,  /* valid request the library does not implement (e.g. d)  */
  TQ_EALIGN = 3,        /* a pointer or stride violates the stated alignment       */
  TQ_ENOMEM = 4,        /* device or host allocation failed (codebook build only)  */
  TQ_EWORKSPACE = 5,    /* workspace missing or smaller than tq_workspace_size     */
  TQ_EDEVICE = 6        /* a HIP runtime call or kernel launch failed              */
} tq_status;

enum { TQ_MSE = 0, TQ_PROD = 1 };                 /* [TQ] "Method"                  */
enum { TQ_F32 = 0, TQ_BF16 = 1 };                 /* element types of x and q       */
enum { TQ_ROT_HAAR = 0, TQ_ROT_GIVEN = 1, TQ_ROT_CALIBRATE = 2, TQ_ROT_HADAMARD = 3 };
enum { TQ_LAYOUT_ROW = 0, TQ_LAYOUT_COL = 1 };

#define TQ_TILE 64          /* vectors per record tile                         */
#define TQ_MAX_BITS 5       /* max index bits per coordinate (32 levels)       */
#define TQ_MAX_LEVELS 32

typedef struct tq_codebook tq_codebook;

/* Description of a codec.
 *   d          dimension; the GPU kernels support d = 128 (KV heads) and any
 *              multiple of 128 up to 4096 for scoring/search (d = 1536 is the
 *              vector-search size).
 *   mode       TQ_MSE: `bits` index bits per coordinate.  TQ_PROD: bits-1 index
 *              bits plus a 1-bit QJL sketch of the residual ([TQ] "Method").
 *   bits       total bits per coordinate (TQ_PROD needs bits >= 2).
 *   bitmap     optional host array [d] of per-dim index bits (1..5) replacing the
 *              uniform bits (SpectralQuant water-filled map, e.g. 5,3,2,2,1,..;
 *              [SQ] tweet 6); NULL = uniform.
 *   qjl_dims   m, TQ_PROD only: the sketch S (m x m, i.i.d. N(0,1)) acts on
 *              rotated dims 0..m-1 ([SQ] tweet 5); 0 means m = d (TurboQuant).
 *   rotation   TQ_ROT_HAAR: Pi is Haar from seed_rotation ([TQ] "Method",
 *              [LK] dense QR); codebooks are Lloyd-Max for the rotated-
 *              coordinate Beta law at dimension d.
 *              TQ_ROT_GIVEN: Pi taken from `given` (host, [num_heads][d][d]
 *              fp32, row i = i-th basis vector), Beta-law codebooks.
 *              TQ_ROT_CALIBRATE: per head, Pi = eigenvectors of the centred
 *              covariance of `calib` ([num_heads][calib_n][d] of
 *              calib_dtype; host, or device with calib_on_device), eigenvalues
 *              descending, each row signed so its
 *              largest-magnitude entry is positive ([SQ] tweet 4); per-dim
 *              codebook = Gaussian Lloyd-Max with b_i levels scaled by sigma_i,
 *              the RMS of rotated coordinate i of the normalised calibration
 *              vectors.
 *              TQ_ROT_HADAMARD: randomized Hadamard rotation ([LK]: the
 *              reference cache's O(d log d) mode; the launch post's summary
 *              "random Hadamard rotation"): Pi = H diag(s) / sqrt(d) with H the
 *              Sylvester Walsh-Hadamard matrix (H[i][j] = (-1)^popcount(i & j))
 *              and s_j = +1 / -1 from bit 0 of word j of the Philox stream 3
 *              of seed_rotation; d must be a power of two; Beta-law codebooks
 *              as for TQ_ROT_HAAR.  At d = 128 it is applied as a fast
 *              Walsh-Hadamard transform by the query rotation (tq_score,
 *              tq_search_topk, tq_decode_attend, tq_decode_step), the inverse
 *              value rotation of the decode output, tq_append, and tq_encode of
 *              bf16 inputs into mse COL 4-bit or prod ROW 2-bit records; the
 *              other encodes use Pi itself.
 *   num_heads  rotations held by the codebook (one per KV head for
 *              TQ_ROT_CALIBRATE / TQ_ROT_GIVEN, or per outlier channel list of
 *              a split codec); TQ_ROT_HAAR otherwise uses 1.
 *   layout     TQ_LAYOUT_ROW or TQ_LAYOUT_COL (COL needs a uniform bit map;
 *              the GPU encode writes COL records for 1, 2 or 4 index bits),
 *              or, for an outlier-channel split, the 2.5-bit mse split (32
 *              outlier channels at outlier_bits 3, the others at bits 2):
 *              per 8-token group, 16 lane blocks (block n: stored
 *              coordinates 16 vb + n, vb = 0..7, each a little-endian word
 *              of 8 codes, 3 bytes for the outlier coordinates (n < 8, vb
 *              even), 2 bytes otherwise), 288 bytes a group, then n_x of the
 *              regular and of the outlier instance; its decode runs on the
 *              MFMA kernel.
 *   seed_*     seeds of the Philox4x32-10 streams of Pi (stream 1; the
 *              Hadamard signs use stream 3) and S (stream 2).
 *   device     HIP device ordinal that holds the codebook's tables.
 *   waterfill_bits  TQ_ROT_CALIBRATE with bitmap NULL only (0 = off): the
 *              per-dim index bits are allocated from the calibration spectrum
 *              by discrete reverse water-filling ([SQ] tweet 6) with
 *              tq_water_fill: waterfill_bits index bits in total, 1..5 per dim,
 *              lambda_i = sigma_i^2 averaged over the heads.
 *   outlier_dims  o, 0 = off.  Outlier-channel split ([TQ] "Method": for the
 *              KV-cache experiments the channels are divided into an outlier
 *              and a regular group, each quantized by its own TurboQuant
 *              instance; 32 channels at 3 bits + 96 at 2 bits is the 2.5-bit
 *              setting).  The regular instance covers the other d - o channels
 *              (ascending) with `bits`, Pi from seed_rotation and S from
 *              seed_sketch; the outlier instance covers outlier_channels (in
 *              list order) with outlier_bits, seeds seed_rotation + 1 and
 *              seed_sketch + 1; both are Haar TurboQuant codecs of `mode` at
 *              their own dimension (Beta-law codebooks at o and d - o, prod
 *              with a full sketch of each instance).  Needs d = 128,
 *              o in {32, 64, 96}, rotation TQ_ROT_HAAR, bitmap NULL,
 *              qjl_dims 0, layout ROW; num_heads >= 1 channel lists.
 *              The codec is held in "stored order": stored coordinate i
 *              (blk = i / 32, r = i % 32, p = o / 4 per block) is outlier
 *              coordinate p blk + r when r < p, else regular coordinate
 *              (32 - p) blk + r - p; the rotation rows, the (block-diagonal)
 *              sketch, the per-dim codebooks, the index bits and the sign bits
 *              all follow that order, and tq_codebook_export returns them so.
 *              Scores: s = sum over the two groups g of
 *              n_x,g (sum_{i in g} q'_i c_i[idx_i]
 *                     + n_r,g sqrt(pi/2)/m_g sum_{j in g} qs_j (2 bit_j - 1)),
 *              m_g the group's size; each group stores its own norms.
 *   outlier_bits   total bits per coordinate of the outlier instance.
 *   outlier_channels  host int32 [num_heads][o]: distinct channels in [0, d)
 *              per head (head h of a multi-head codec uses row h).
 *   calib_on_device  TQ_ROT_CALIBRATE: 0 = `calib` is a host array and the
 *              calibration runs on the host; 1 = `calib` is a device array on
 *              `device` (same shape and dtype) and the O(calib_n d^2) part of
 *              the calibration runs there: per head the fp64 column sums,
 *              second moment and second moment of the normalised vectors
 *              ([SQ] tweet 4: the short calibration pass); the d x d
 *              eigensolves and the codebooks stay on the host.  Needs d a
 *              multiple of 32 and device >= 0.
 */
typedef struct {
  int32_t d;
  int32_t mode;
  int32_t bits;
  const uint8_t* bitmap;
  int32_t qjl_dims;
  int32_t rotation;
  int32_t num_heads;
  int32_t layout;
  uint64_t seed_rotation;
  uint64_t seed_sketch;
  const float* given;
  const void* calib;
  int64_t calib_n;
  int32_t calib_dtype;
  int32_t device;
  int32_t waterfill_bits;
  int32_t outlier_dims;
  int32_t outlier_bits;
  const int32_t* outlier_channels;
  int32_t calib_on_device;
} tq_codebook_desc;

/* Sizes of a codec's records. */
typedef struct {
  int32_t d, mode, m, layout, num_heads, uniform;
  int32_t index_bits_total;   /* B = sum of per-dim index bits                 */
  int32_t code_bytes;         /* per vector, ceil(B/8)                          */
  int32_t sign_bytes;         /* per vector, ceil(m/8) (0 for mse)              */
  int32_t norms;              /* fp16 norms per vector: 1 (mse) or 2 (prod), x2 split */
  int64_t tile_bytes;         /* bytes of one 64-vector tile                    */
  int64_t off_signs, off_nx, off_nr;  /* byte offsets of the fields in a tile  */
  int32_t outlier_dims;       /* o of a split codec, else 0                    */
  int32_t outlier_per_block;  /* o / 4: outlier coordinates per 32 stored ones */
  int64_t off_nx_o, off_nr_o; /* split: outlier instance's norms, else -1      */
} tq_codebook_info;

/* Build a codebook (host math once, then device tables on desc->device).
 * Synchronous.  [TQ] "Method": codebooks are solved once, offline. */
tq_status tq_codebook_build(const tq_codebook_desc* desc, tq_codebook** out);
tq_status tq_codebook_free(tq_codebook* cb);

/* Append-on-decode (d = 128): encode one new vector per (sequence, head) into
 * its existing records, at token index positions[b] of sequence b.
 * TurboQuant also quantizes the tokens generated during decoding (TurboQuant
 * paper review, "Comparison"); this call writes them in place, so the next
 * tq_decode_attend (with seq_lens advanced past them) reads them like any
 * other token.
 *   x          device [B][H][d] new vectors (fp32 or bf16), last dim
 *              contiguous, strides xs_b, xs_h in elements; head h is encoded
 *              with rotation head h of a multi-head codebook.
 *   records    device; the records of (b, h) start at records + b * rs_b +
 *              h * rs_h bytes and hold `capacity` tokens (their tile count).
 *   positions  device int32 [B]; entries outside [0, capacity) are skipped.
 * Supported: ROW records of any bit map (mse, or prod with m <= d), COL
 * records of uniform mse codecs with 1, 2 or 4 index bits and of the 2.5-bit
 * split mse codec; TQ_EUNSUPPORTED otherwise.  Only the new slot's bytes (COL: the new vector's bits in each
 * dim's field) change.  Calls for the same records must not overlap.
 * Errors: TQ_EINVAL (null pointer, negative size, bad dtype), TQ_EALIGN
 * (records or record strides not 4-byte aligned), TQ_EDEVICE (launch). */
tq_status tq_append(const tq_codebook* cb, const void* x, int32_t x_dtype, int32_t B, int32_t H,
                    int64_t xs_b, int64_t xs_h, void* records, int64_t rs_b, int64_t rs_h,
                    const int32_t* positions, int32_t capacity, void* stream);

/* Discrete reverse water-filling of index bits over dimensions with variances
 * lambda ([SQ] tweet 6: water-filling of the bits over the dominant dims,
 * after Shannon and Berger).  Host only; no device work.
 *   lambda      host [d] variances (>= 0) of the rotated coordinates.
 *   total_bits  index bits to hand out, d*min_bits <= total_bits <= d*max_bits.
 *   min_bits, max_bits  per-dim range, 1 <= min_bits <= max_bits <= 5.
 *   bits_out    host [d], written.
 * Every dim starts at min_bits; then, one bit at a time, the dim with the
 * largest drop lambda_i (D(b_i) - D(b_i + 1)) of its distortion gets the bit,
 * D(b) being the mean squared error of the b-bit Lloyd-Max quantizer of the
 * standard normal law (ties to the lower dim).  D is convex in b, so this
 * greedy allocation minimises sum_i lambda_i D(b_i) under the budget.
 * TQ_EINVAL on a null pointer, d < 1, a negative lambda or a budget or range
 * outside the bounds above. */
tq_status tq_water_fill(const double* lambda, int32_t d, int32_t total_bits, int32_t min_bits,
                        int32_t max_bits, uint8_t* bits_out);
tq_status tq_codebook_get_info(const tq_codebook* cb, tq_codebook_info* info);

/* Copy a codebook's parameters to host memory (any pointer may be NULL):
 *   rot [d][d] fp32 of head `head`; sketch [m][m] fp32;
 *   centroids [d][TQ_MAX_LEVELS] and boundaries [d][TQ_MAX_LEVELS-1] fp64 of
 *   head `head` (unused entries 0); levels [d] = 2^(bits of dim i).
 *   The fp64 values are those of the Lloyd-Max solution; kernels use them
 *   rounded to fp32. */
tq_status tq_codebook_export(const tq_codebook* cb, int32_t head, float* rot, float* sketch,
                             double* centroids, double* boundaries, int32_t* levels);

/* Bytes of the record tiles holding n vectors. */
int64_t tq_records_bytes(const tq_codebook* cb, int64_t n);

/* Encode a batch of vector sets.  [TQ] "Method": n_x = ||x||, y = Pi x/n_x,
 * idx_i = #{boundaries t of dim i with t <= y_i}, so a y_i exactly on a
 * boundary goes to the upper cell -- except in the d = 128 kernels of uniform
 * codecs: with 2 index bits they compare |y_i| with the positive boundary
 * (the codebook is symmetric) and put a negative y_i exactly on a boundary
 * into the lower cell, the one of larger magnitude; with 4 index bits in the
 * COL layout they compare y_i with the boundary of its bucket in bucket units
 * (y_i / w + offset, rounded to fp32), which decides as the exact comparison
 * except within about 1e-7 of a boundary (all readings agree everywhere off
 * the boundaries); prod:
 * r = y - c[idx] on dims 0..m-1, n_r = ||r||, bit_j = [(S r)_j >= 0].  A zero
 * vector encodes y = 0 and stores n_x = 0.
 *   x        device, element (b, h, t, i) at x[b*xs_b + h*xs_h + t*xs_t + i] of
 *            type x_dtype (TQ_F32 or TQ_BF16); row starts 16-byte aligned.
 *   batch, heads, tokens   sizes; `heads` indexes the codebook's rotation when
 *            it holds num_heads > 1 (must then equal num_heads).
 *   records  device; the tiles of set (b, h) start at
 *            records + b*rs_b + h*rs_h bytes (16-byte aligned) and hold
 *            ceil(tokens/64) tiles.
 *   workspace device scratch of tq_workspace_size(cb, TQ_OP_ENCODE, 0, 0, 0)
 *            bytes (0 for d = 128: may be NULL).
 * Supported: d = 128 (fused kernel, any codec) and d a multiple of 128 up to
 * 4096 with a uniform ROW codec (GEMM-based path, rows in chunks). */
tq_status tq_encode(const tq_codebook* cb, const void* x, int32_t x_dtype, int64_t batch,
                    int64_t heads, int64_t tokens, int64_t xs_b, int64_t xs_h, int64_t xs_t,
                    void* records, int64_t rs_b, int64_t rs_h, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Keys and values of the same tokens encoded together, as a KV cache is
 * written ([TQ] "Method", KV-cache setting: every new token's key and value
 * are quantized online, each by its own codec).  The result is that of
 * tq_encode(kcb, k, ...) followed by tq_encode(vcb, v, ...), byte for byte:
 *   k, v     device rows of x_dtype with the same sizes and strides
 *            (xs_b, xs_h, xs_t as for tq_encode);
 *   k_records, v_records  device records of each codec, set (b, h) at
 *            k_records + b*kr_b + h*kr_h (likewise v), 16-byte aligned.
 * Both codecs must be d = 128 (else TQ_EUNSUPPORTED) on one device (else
 * TQ_EINVAL); the other errors are tq_encode's, checked for both before any
 * launch.  bf16 rows with a TurboQuant-prod 3-bit ROW key codec and a
 * TurboQuant-mse 4-bit COL value codec (dense Pi) run as one launch whose
 * workgroups take the value tiles as soon as the key tiles leave CUs free;
 * every other pair runs as the two encodes.  No workspace is needed. */
tq_status tq_encode_kv(const tq_codebook* kcb, const tq_codebook* vcb, const void* k, const void* v,
                       int32_t x_dtype, int64_t batch, int64_t heads, int64_t tokens, int64_t xs_b,
                       int64_t xs_h, int64_t xs_t, void* k_records, int64_t kr_b, int64_t kr_h,
                       void* v_records, int64_t vr_b, int64_t vr_h, void* stream);

/* Inner-product scores of nq queries against n ROW records of head `head`:
 *   scores[i][t] = n_x (sum_j q'_j c[idx_j] + n_r sqrt(pi/2)/m sum_j qs_j (2 bit_j - 1)),
 *   q' = Pi q, qs = S q'[0:m] ([TQ] "Method"; estimator of <q, x>).
 *   q        device fp32 [nq][d];  scores device fp32 [nq][n].
 *   workspace >= tq_workspace_size(cb, TQ_OP_SCORE, nq, n, 0) bytes (device).
 * Supported: d = 128 (any ROW codec) and d a multiple of 128 up to 4096 with a
 * uniform codec (full sketch for prod); else TQ_EUNSUPPORTED.  More than
 * 261632 queries run as consecutive passes of that many, sharing the
 * workspace (whose size then covers one pass). */
tq_status tq_score(const tq_codebook* cb, const float* q, int64_t nq, int32_t head,
                   const void* records, int64_t n, float* scores, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Compressed KV cache of one layer, records as written by tq_encode.
 * Contiguous layout (block_table NULL): set (b, h) of the keys starts at
 * k_records + b*k_stride_seq + h*k_stride_head bytes; likewise for values.
 * Paged layout (block_table non-NULL): k_records and v_records are pools of
 * pages, each page_tiles record tiles (64 tokens per tile) of the codec; tile
 * t of set (b, h) is tile t % page_tiles of page
 * block_table[(b*Hkv + h)*max_pages + t / page_tiles] (a page index into the
 * pool; keys and values use the same index in their own pools) and the
 * strides are not used.  Only the entries of tiles below seq_lens[b] (below
 * max_tokens without seq_lens; tq_decode_step: through slot seq_lens[b]) are
 * read.  A page holds whole tiles, so tq_encode can fill it
 * directly (records = the page, tokens = a multiple of 64 * page_tiles, or
 * the set's tail). */
typedef struct {
  const void* k_records;
  const void* v_records;
  int64_t k_stride_seq, k_stride_head;
  int64_t v_stride_seq, v_stride_head;
  int32_t max_tokens;         /* tokens stored per (b, h)                       */
  const int32_t* seq_lens;    /* device [B] valid tokens per sequence, or NULL  */
  const int32_t* block_table; /* device [B*Hkv][max_pages] page indices, or NULL */
  int32_t page_tiles;         /* tiles per page (paged layout), >= 1            */
  int32_t max_pages;          /* entries per (b, h) row of block_table          */
} tq_kv_view;

/* One decode step of grouped-query attention over a compressed cache ([TQ]
 * "Sparks": rotation and codebook lookup fused into attention):
 *   logit_{b,h,t} = softmax_scale * score(q_{b,h}, k_{b,g,t}), g = h / (Hq/Hkv),
 *   out_{b,h} = sum_t softmax_t(logit) * v_hat_{b,g,t},
 *   v_hat = n_v Pi_v^T c_v[idx] (mse reconstruction of the value).
 *   kcb      ROW codec of the keys (num_heads 1 or Hkv);
 *   vcb      mse codec of the values (num_heads 1 or Hkv), d = 128: COL records
 *            of a uniform codec with up to 4 index bits, or ROW records of a
 *            uniform codec or of an outlier-channel split one (each stored
 *            coordinate scaled by its group's norm; [TQ] "Method": the
 *            KV-cache experiments split the channels of keys and values);
 *            other value codecs give TQ_EUNSUPPORTED.
 *   q        device [B][Hq][d] of q_dtype;  out device fp32 [B][Hq][d].
 *   workspace >= tq_workspace_size(kcb, TQ_OP_DECODE, B*Hq, max_tokens, Hkv). */
/* A sequence with no tokens (seq_lens[b] = 0, or max_tokens = 0) gets an
 * all-zero output; with max_tokens = 0 no record, block-table entry or
 * workspace byte is read. */
tq_status tq_decode_attend(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                           int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                           const tq_kv_view* kv, float softmax_scale, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* tq_decode_attend without any allocation, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid it).  The workspace is a device array inside the library, of
 * TQ_NOALLOC_SCRATCH_BYTES on every GPU the library runs on (held until the
 * process ends); its address is looked up on the first call for a device.
 * Arguments, results and errors are those of tq_decode_attend, and
 * TQ_EWORKSPACE when tq_workspace_size(kcb, TQ_OP_DECODE, B*Hq, max_tokens,
 * Hkv) exceeds TQ_NOALLOC_SCRATCH_BYTES.  The call itself allocates nothing.
 * All calls on one GPU share its array: calls that overlap on one GPU race
 * (issue them on one stream, or order them). */
#define TQ_NOALLOC_SCRATCH_BYTES (32u << 20)
tq_status tq_decode_attend_noalloc(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                                   int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                   const tq_kv_view* kv, float softmax_scale, float* out, void* stream);

/* One decode step with append-on-decode (TurboQuant paper review,
 * "Comparison": the tokens generated during decoding are quantized too):
 * the new key and value of every (sequence, KV head) are encoded into slot
 * seq_lens[b] of its records (as tq_append), then the step attends over
 * seq_lens[b] + 1 tokens (as tq_decode_attend).  seq_lens is required and is
 * not changed (the caller advances it); a sequence whose slot seq_lens[b] is
 * not below max_tokens gets no new token and attends over max_tokens.
 *   k_new, v_new  device [B][Hkv][d] of new_dtype (TQ_F32 or TQ_BF16), rows
 *            contiguous.
 *   kv       contiguous or paged view; its records are written (the new
 *            slots only), so they must be device memory the caller owns.
 * The codecs, q, out and workspace are as for tq_decode_attend; the key and
 * value codecs must also be ones tq_append supports.  Errors: those of
 * tq_decode_attend and tq_append, and TQ_EINVAL when seq_lens is NULL. */
tq_status tq_decode_step(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                         int32_t q_dtype, const void* k_new, const void* v_new, int32_t new_dtype,
                         int32_t B, int32_t Hq, int32_t Hkv, const tq_kv_view* kv,
                         float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Top-k inner-product search over n ROW records ([TQ] "Validation": vector
 * search with TurboQuant codes).  For each query the k largest scores
 * (as tq_score), descending; equal scores go to the smaller id.
 *   top_scores device fp32 [nq][k]; top_ids device int64 [nq][k]; 1 <= k <= 16.
 *   workspace >= tq_workspace_size(cb, TQ_OP_TOPK, nq, n, k); more than
 *   65408 queries run as consecutive passes of that many, sharing it. */
tq_status tq_search_topk(const tq_codebook* cb, const float* q, int64_t nq,
                         const void* records, int64_t n, int32_t k, float* top_scores,
                         int64_t* top_ids, void* workspace, size_t workspace_bytes,
                         void* stream);

enum { TQ_OP_SCORE = 0, TQ_OP_DECODE = 1, TQ_OP_TOPK = 2, TQ_OP_ENCODE = 3 };

/* Device workspace bytes an operation needs (0 on bad arguments or when none
 * is needed):  TQ_OP_SCORE (a = nq, b = n), TQ_OP_DECODE (a = B*Hq,
 * b = max_tokens, c = Hkv), TQ_OP_TOPK (a = nq, b = n, c = k),
 * TQ_OP_ENCODE (no size arguments). */
size_t tq_workspace_size(const tq_codebook* cb, int32_t op, int64_t a, int64_t b, int64_t c);

const char* tq_status_string(tq_status s);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
