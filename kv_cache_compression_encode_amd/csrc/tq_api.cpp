// C-ABI layer of the codec library: argument validation, codebook build
// (host math + device tables) and kernel dispatch.  Every check runs before
// any launch; errors return a tq_status and leave outputs untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>
#include <thread>

#include "tq_internal.h"
#include "tq_kernels.h"

using namespace tq;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// f(h) for h < heads, spread over host threads (one per head up to the
// hardware's count).  False if any call ran out of memory.
template <class F>
bool for_each_head(int heads, F&& f) {
  std::atomic<bool> ok{true};
  auto run = [&](int h) {
    try {
      f(h);
    } catch (const std::bad_alloc&) {
      ok = false;
    }
  };
  const int nth = std::max(1, std::min<int>(heads, int(std::thread::hardware_concurrency())));
  if (nth == 1) {
    for (int h = 0; h < heads; ++h) run(h);
  } else {
    std::vector<std::thread> pool;
    for (int w = 0; w < nth; ++w)
      pool.emplace_back([&, w] {
        for (int h = w; h < heads; h += nth) run(h);
      });
    for (std::thread& t : pool) t.join();
  }
  return ok;
}

// The calibration moments on the device (calib_on_device): per head the
// column sums, sum_t x x^T and sum_t x x^T / ||x||^2, fp64, copied back.
tq_status device_moments(const tq_codebook_desc& ds, int heads, std::vector<double>& mom_x,
                         std::vector<double>& mom_u, std::vector<double>& sum_x) {
  const int d = ds.d;
  const int64_t n = ds.calib_n;
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (hipSetDevice(ds.device) != hipSuccess) return TQ_EDEVICE;
  const size_t dd = size_t(heads) * d * d, hd = size_t(heads) * d;
  double* buf = nullptr;
  tq_status st = TQ_OK;
  if (hipMalloc(reinterpret_cast<void**>(&buf), (2 * dd + hd + size_t(heads) * n) * sizeof(double)) != hipSuccess) {
    st = TQ_ENOMEM;
  } else {
    double *mx = buf, *mu = mx + dd, *sx = mu + dd, *rinv2 = sx + hd;
    if (launch_calib_moments(ds.calib, ds.calib_dtype == TQ_BF16, heads, n, d, rinv2, mx, mu, sx, nullptr) !=
            hipSuccess ||
        hipMemcpy(mom_x.data(), mx, dd * sizeof(double), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(mom_u.data(), mu, dd * sizeof(double), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(sum_x.data(), sx, hd * sizeof(double), hipMemcpyDeviceToHost) != hipSuccess)
      st = TQ_EDEVICE;
    (void)hipFree(buf);
  }
  (void)hipSetDevice(prev);
  return st;
}

template <class T>
tq_status upload(T** dst, const T* src, size_t count) {
  if (hipMalloc(reinterpret_cast<void**>(dst), count * sizeof(T)) != hipSuccess) return TQ_ENOMEM;
  if (hipMemcpy(*dst, src, count * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return TQ_EDEVICE;
  return TQ_OK;
}

void free_device(tq_codebook* cb) {
  DeviceTables& t = cb->dev;
  void* ptrs[] = {t.rot, t.rot_t, t.rot_hi, t.rot_lo, t.sketch, t.sketch_t, t.sketch_hi,
                  t.sketch_lo, t.thr, t.cen, t.bitpos, t.dim_bits, t.sq_tail, t.sq_gm, t.had_mask,
                  t.had_sign, t.omask, t.rot_tiles, t.sk_tiles};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  t = DeviceTables{};
}

void fill_info(tq_codebook* cb) {
  tq_codebook_info& in = cb->info;
  const int d = cb->desc.d;
  in.d = d;
  in.mode = cb->desc.mode;
  in.m = cb->m;
  in.layout = cb->desc.layout;
  in.num_heads = int(cb->rot32.size() / (size_t(d) * d));
  in.uniform = cb->uniform ? 1 : 0;
  int total = 0;
  for (uint8_t b : cb->bits) total += b;
  in.index_bits_total = total;
  in.code_bytes = (total + 7) / 8;
  in.sign_bytes = cb->desc.mode == TQ_PROD ? (cb->m + 7) / 8 : 0;
  in.norms = cb->desc.mode == TQ_PROD ? 2 : 1;
  int64_t off = 0;
  off += int64_t(kTile) * in.code_bytes;  // both layouts: 64 vectors x code bytes
  in.off_signs = off;
  off += int64_t(kTile) * in.sign_bytes;
  in.off_nx = off;
  off += 2 * kTile;
  in.off_nr = cb->desc.mode == TQ_PROD ? off : -1;
  if (cb->desc.mode == TQ_PROD) off += 2 * kTile;
  in.outlier_dims = cb->outlier;
  in.outlier_per_block = cb->outlier ? cb->outlier * 32 / d : 0;
  in.off_nx_o = in.off_nr_o = -1;
  if (cb->outlier) {
    in.norms *= 2;
    in.off_nx_o = off;
    off += 2 * kTile;
    if (cb->desc.mode == TQ_PROD) {
      in.off_nr_o = off;
      off += 2 * kTile;
    }
  }
  in.tile_bytes = off;
}

// Outlier-channel split: two Haar TurboQuant instances (outlier channels with
// outlier_bits, the others with bits) held as one codec in stored order.
// Stored coordinate i = 32 blk + r is outlier coordinate p blk + r for r < p
// (p = o / 4), else regular coordinate (32 - p) blk + r - p.  Rotation row i
// is that instance's Pi row placed on its channels; the sketch is
// block-diagonal (S_o on outlier pairs, S_r on regular pairs, zero across).
tq_status build_split(tq_codebook* cb, const tq_codebook_desc& ds) {
  const int d = ds.d, o = ds.outlier_dims;
  if (d != 128) return TQ_EUNSUPPORTED;
  if (o != 32 && o != 64 && o != 96) return TQ_EUNSUPPORTED;
  if (!ds.outlier_channels || ds.bitmap || ds.waterfill_bits > 0 || ds.rotation != TQ_ROT_HAAR)
    return TQ_EINVAL;
  if (ds.qjl_dims != 0 && ds.qjl_dims != d) return TQ_EUNSUPPORTED;
  const int heads = std::max(1, ds.num_heads);
  const int ub_r = ds.mode == TQ_PROD ? ds.bits - 1 : ds.bits;
  const int ub_o = ds.mode == TQ_PROD ? ds.outlier_bits - 1 : ds.outlier_bits;
  if (ub_r < 1 || ub_r > kMaxBits || ub_o < 1 || ub_o > kMaxBits) return TQ_EINVAL;
  // col records: the 2.5-bit split of mse values only (32 outlier channels
  // at 3 index bits, 96 at 2), whose 8-token code words the MFMA decode reads
  if (ds.layout == TQ_LAYOUT_COL && (ds.mode != TQ_MSE || o != 32 || ub_o != 3 || ub_r != 2))
    return TQ_EUNSUPPORTED;
  if (ds.layout != TQ_LAYOUT_ROW && ds.layout != TQ_LAYOUT_COL) return TQ_EINVAL;
  // channel lists: outlier channels in list order, the others ascending
  std::vector<int> och(size_t(heads) * o), rch(size_t(heads) * (d - o));
  for (int h = 0; h < heads; ++h) {
    std::vector<char> seen(d, 0);
    for (int k = 0; k < o; ++k) {
      const int c = ds.outlier_channels[size_t(h) * o + k];
      if (c < 0 || c >= d || seen[c]) return TQ_EINVAL;
      seen[c] = 1;
      och[size_t(h) * o + k] = c;
    }
    int k = 0;
    for (int c = 0; c < d; ++c)
      if (!seen[c]) rch[size_t(h) * (d - o) + k++] = c;
  }
  const int p = o * 32 / d;
  std::vector<int> grp(d), crd(d);
  for (int i = 0; i < d; ++i) {
    const int blk = i / 32, r = i % 32;
    grp[i] = r < p ? 1 : 0;
    crd[i] = r < p ? p * blk + r : (32 - p) * blk + r - p;
  }
  cb->outlier = o;
  cb->omask.assign(size_t(heads) * (d / 32), 0u);
  for (int h = 0; h < heads; ++h)
    for (int k = 0; k < o; ++k) {
      const int c = och[size_t(h) * o + k];
      cb->omask[size_t(h) * (d / 32) + c / 32] |= 1u << (c % 32);
    }
  cb->uniform = false;
  cb->ubits = 0;
  cb->m = ds.mode == TQ_PROD ? d : 0;
  cb->bits.assign(d, 0);
  for (int i = 0; i < d; ++i) cb->bits[i] = uint8_t(grp[i] ? ub_o : ub_r);
  // rotations: Pi_o (seed_rotation + 1) and Pi_r (seed_rotation), stream 1
  const int dims[2] = {d - o, o};
  std::vector<double> pi[2];
  for (int gsel = 0; gsel < 2; ++gsel) {
    const int n = dims[gsel];
    std::vector<double> g(size_t(n) * n);
    philox_normals(ds.seed_rotation + uint64_t(gsel), 1, int64_t(n) * n, g.data());
    pi[gsel].resize(size_t(n) * n);
    haar_from_gaussian(n, g.data(), pi[gsel].data());
  }
  cb->rot64.assign(size_t(heads) * d * d, 0.0);
  for (int h = 0; h < heads; ++h)
    for (int i = 0; i < d; ++i) {
      const int gsel = grp[i], n = dims[gsel];
      const int* ch = gsel ? &och[size_t(h) * o] : &rch[size_t(h) * (d - o)];
      for (int k = 0; k < n; ++k) cb->rot64[(size_t(h) * d + i) * d + ch[k]] = pi[gsel][size_t(crd[i]) * n + k];
    }
  cb->rot32.resize(cb->rot64.size());
  for (size_t e = 0; e < cb->rot64.size(); ++e) cb->rot32[e] = float(cb->rot64[e]);
  // sketches: S_o (seed_sketch + 1) and S_r (seed_sketch), stream 2, fp16 values
  if (ds.mode == TQ_PROD) {
    std::vector<float> sk[2];
    for (int gsel = 0; gsel < 2; ++gsel) {
      const int n = dims[gsel];
      std::vector<double> s(size_t(n) * n);
      philox_normals(ds.seed_sketch + uint64_t(gsel), 2, int64_t(n) * n, s.data());
      sk[gsel].resize(s.size());
      for (size_t e = 0; e < s.size(); ++e) sk[gsel][e] = f16_to_f32(f32_to_f16_rne(float(s[e])));
    }
    cb->sketch32.assign(size_t(d) * d, 0.f);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j)
        if (grp[i] == grp[j])
          cb->sketch32[size_t(i) * d + j] = sk[grp[i]][size_t(crd[i]) * dims[grp[i]] + crd[j]];
  }
  // per-dim Beta-law codebooks of each instance's dimension
  const LloydMaxResult books[2] = {lloyd_max_sphere(d - o, ub_r), lloyd_max_sphere(o, ub_o)};
  cb->cen64.assign(size_t(heads) * d * kMaxLevels, 0.0);
  cb->thr64.assign(size_t(heads) * d * (kMaxLevels - 1), 0.0);
  cb->cen32.assign(size_t(heads) * d * kMaxLevels, 0.f);
  cb->thr32.assign(size_t(heads) * d * kMaxLevels, INFINITY);
  for (int h = 0; h < heads; ++h)
    for (int i = 0; i < d; ++i) {
      const LloydMaxResult& lm = books[grp[i]];
      const int L = 1 << cb->bits[i];
      for (int k = 0; k < L; ++k) {
        cb->cen64[(size_t(h) * d + i) * kMaxLevels + k] = lm.centroids[k];
        cb->cen32[(size_t(h) * d + i) * kMaxLevels + k] = float(lm.centroids[k]);
      }
      for (int k = 0; k + 1 < L; ++k) {
        cb->thr64[(size_t(h) * d + i) * (kMaxLevels - 1) + k] = lm.boundaries[k];
        cb->thr32[(size_t(h) * d + i) * kMaxLevels + k] = float(lm.boundaries[k]);
      }
    }
  cb->bitpos.assign(size_t(kMaxBits) * d, -1);
  int pos = 0;
  for (int pl = 0; pl < kMaxBits; ++pl)
    for (int i = 0; i < d; ++i)
      if (cb->bits[i] > pl) cb->bitpos[size_t(pl) * d + i] = int16_t(pos++);
  fill_info(cb);
  cb->info.num_heads = heads;
  return TQ_OK;
}

tq_status build_host(tq_codebook* cb, const tq_codebook_desc& ds) {
  if (ds.outlier_dims != 0) return ds.outlier_dims < 0 ? TQ_EINVAL : build_split(cb, ds);
  const int d = ds.d;
  // ---------------------------------------------------------------- bits
  cb->bits.assign(d, 0);
  const int ub = ds.mode == TQ_PROD ? ds.bits - 1 : ds.bits;
  const bool waterfill = ds.waterfill_bits > 0;
  if (waterfill) {
    // allocated from the calibration spectrum once the rotation is known
    if (ds.bitmap || ds.rotation != TQ_ROT_CALIBRATE) return TQ_EINVAL;
    if (ds.waterfill_bits < d || ds.waterfill_bits > d * kMaxBits) return TQ_EINVAL;
    std::fill(cb->bits.begin(), cb->bits.end(), uint8_t(1));
  } else if (ds.bitmap) {
    for (int i = 0; i < d; ++i) {
      if (ds.bitmap[i] < 1 || ds.bitmap[i] > kMaxBits) return TQ_EINVAL;
      cb->bits[i] = ds.bitmap[i];
    }
  } else {
    if (ub < 1 || ub > kMaxBits) return TQ_EINVAL;
    std::fill(cb->bits.begin(), cb->bits.end(), uint8_t(ub));
  }
  cb->uniform = std::all_of(cb->bits.begin(), cb->bits.end(), [&](uint8_t b) { return b == cb->bits[0]; });
  cb->ubits = cb->uniform ? cb->bits[0] : 0;
  if (ds.layout == TQ_LAYOUT_COL && !cb->uniform) return TQ_EUNSUPPORTED;
  cb->m = ds.mode == TQ_PROD ? (ds.qjl_dims > 0 ? ds.qjl_dims : d) : 0;
  if (cb->m > d) return TQ_EINVAL;

  // ----------------------------------------------------------- rotations
  int heads = 1;
  std::vector<double> mom_u;  // calibration on the device: sum_t u u^T per head
  if (ds.rotation == TQ_ROT_HAAR) {
    std::vector<double> g(size_t(d) * d);
    philox_normals(ds.seed_rotation, 1, int64_t(d) * d, g.data());
    cb->rot64.resize(size_t(d) * d);
    haar_from_gaussian(d, g.data(), cb->rot64.data());
  } else if (ds.rotation == TQ_ROT_HADAMARD) {
    // Pi = H diag(s) / sqrt(d): H Sylvester Walsh-Hadamard, s_j from bit 0 of
    // word j of the Philox stream 3 (block j / 4, word j % 4)
    if (d & (d - 1)) return TQ_EUNSUPPORTED;
    cb->hsign.assign(d, 1);
    const uint32_t key[2] = {uint32_t(ds.seed_rotation), uint32_t(ds.seed_rotation >> 32)};
    for (int blk = 0; blk * 4 < d; ++blk) {
      const uint32_t ctr[4] = {uint32_t(blk), 0u, 3u, 0u};
      uint32_t w[4];
      philox4x32_10(ctr, key, w);
      for (int k = 0; k < 4 && blk * 4 + k < d; ++k) cb->hsign[blk * 4 + k] = (w[k] & 1u) ? -1 : 1;
    }
    cb->rot64.resize(size_t(d) * d);
    const double inv = 1.0 / std::sqrt(double(d));
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j)
        cb->rot64[size_t(i) * d + j] = ((__builtin_popcount(unsigned(i & j)) & 1) ? -inv : inv) * cb->hsign[j];
  } else if (ds.rotation == TQ_ROT_GIVEN) {
    if (!ds.given) return TQ_EINVAL;
    heads = std::max(1, ds.num_heads);
    cb->rot64.assign(ds.given, ds.given + size_t(heads) * d * d);
  } else if (ds.rotation == TQ_ROT_CALIBRATE) {
    if (!ds.calib || ds.calib_n < 2) return TQ_EINVAL;
    if (ds.calib_dtype != TQ_F32 && ds.calib_dtype != TQ_BF16) return TQ_EINVAL;
    heads = std::max(1, ds.num_heads);
    cb->rot64.resize(size_t(heads) * d * d);
    const double nn = double(ds.calib_n);
    std::vector<double> cov(size_t(heads) * d * d);
    if (ds.calib_on_device) {
      if (d % 32 != 0 || ds.device < 0) return TQ_EINVAL;
      std::vector<double> sum_x(size_t(heads) * d);
      mom_u.resize(size_t(heads) * d * d);
      const tq_status ms = device_moments(ds, heads, cov, mom_u, sum_x);
      if (ms != TQ_OK) return ms;
      // centred covariance: sum_t x x^T / n - mean mean^T
      for (int h = 0; h < heads; ++h)
        for (int i = 0; i < d; ++i)
          for (int k = 0; k < d; ++k) {
            double& c = cov[(size_t(h) * d + i) * d + k];
            c = c / nn - (sum_x[size_t(h) * d + i] / nn) * (sum_x[size_t(h) * d + k] / nn);
          }
    } else {
      const bool ok = for_each_head(heads, [&](int h) {
        std::vector<double> x(size_t(ds.calib_n) * d), mean(d, 0.0);
        for (int64_t t = 0; t < ds.calib_n; ++t)
          for (int i = 0; i < d; ++i) {
            const size_t e = (size_t(h) * ds.calib_n + t) * d + i;
            x[size_t(t) * d + i] = ds.calib_dtype == TQ_F32
                                       ? double(static_cast<const float*>(ds.calib)[e])
                                       : double(bf16_to_f32(static_cast<const uint16_t*>(ds.calib)[e]));
          }
        for (int64_t t = 0; t < ds.calib_n; ++t)
          for (int i = 0; i < d; ++i) mean[i] += x[size_t(t) * d + i];
        for (int i = 0; i < d; ++i) mean[i] /= nn;
        double* cv = &cov[size_t(h) * d * d];
        for (int64_t t = 0; t < ds.calib_n; ++t) {
          const double* r = &x[size_t(t) * d];
          for (int i = 0; i < d; ++i) {
            const double a = r[i] - mean[i];
            for (int k = 0; k < d; ++k) cv[size_t(i) * d + k] += a * (r[k] - mean[k]);
          }
        }
        for (size_t e = 0; e < size_t(d) * d; ++e) cv[e] /= nn;
      });
      if (!ok) return TQ_ENOMEM;
    }
    // the d x d eigensolves, one host thread per head
    const bool ok = for_each_head(heads, [&](int h) {
      std::vector<double> lam(d);
      symmetric_eigen(d, &cov[size_t(h) * d * d], lam.data(), &cb->rot64[size_t(h) * d * d]);
    });
    if (!ok) return TQ_ENOMEM;
  } else {
    return TQ_EINVAL;
  }
  cb->rot32.resize(cb->rot64.size());
  for (size_t e = 0; e < cb->rot64.size(); ++e) cb->rot32[e] = float(cb->rot64[e]);

  // -------------------------------------------------------------- sketch
  if (ds.mode == TQ_PROD) {
    std::vector<double> s(size_t(cb->m) * cb->m);
    philox_normals(ds.seed_sketch, 2, int64_t(cb->m) * cb->m, s.data());
    cb->sketch32.resize(s.size());
    // S is stored in fp16 (the draws rounded to fp32, then to fp16): its
    // products on fp16 MFMA are then exact and need no low part
    for (size_t e = 0; e < s.size(); ++e) cb->sketch32[e] = f16_to_f32(f32_to_f16_rne(float(s[e])));
  }

  // ------------------------------------------------ calibration spectrum
  // sigma_i (per head): RMS of rotated coordinate i of the normalised
  // calibration vectors
  std::vector<double> sig(size_t(heads) * d, 1.0);
  if (ds.rotation == TQ_ROT_CALIBRATE && !mom_u.empty()) {
    // from the device moments: sigma_i^2 = p_i^T (sum_t u u^T) p_i / n
    const bool ok = for_each_head(heads, [&](int h) {
      const double* M = &mom_u[size_t(h) * d * d];
      std::vector<double> p(d), w(d);
      for (int i = 0; i < d; ++i) {
        for (int k = 0; k < d; ++k) p[k] = double(cb->rot32[(size_t(h) * d + i) * d + k]);
        for (int j = 0; j < d; ++j) {
          double acc = 0;
          for (int k = 0; k < d; ++k) acc += M[size_t(j) * d + k] * p[k];
          w[j] = acc;
        }
        double v = 0;
        for (int j = 0; j < d; ++j) v += p[j] * w[j];
        sig[size_t(h) * d + i] = std::sqrt(std::max(v, 0.0) / double(ds.calib_n));
      }
    });
    if (!ok) return TQ_ENOMEM;
  } else if (ds.rotation == TQ_ROT_CALIBRATE) {
    std::vector<double> acc(d), u(d);
    for (int h = 0; h < heads; ++h) {
      std::fill(acc.begin(), acc.end(), 0.0);
      const float* p = &cb->rot32[size_t(h) * d * d];
      for (int64_t t = 0; t < ds.calib_n; ++t) {
        double nn = 0;
        for (int i = 0; i < d; ++i) {
          const size_t e = (size_t(h) * ds.calib_n + t) * d + i;
          u[i] = ds.calib_dtype == TQ_F32 ? double(static_cast<const float*>(ds.calib)[e])
                                          : double(bf16_to_f32(static_cast<const uint16_t*>(ds.calib)[e]));
          nn += u[i] * u[i];
        }
        nn = std::sqrt(nn);
        for (int i = 0; i < d; ++i) u[i] = nn > 0 ? u[i] / nn : 0.0;
        for (int i = 0; i < d; ++i) {
          double y = 0;
          for (int k = 0; k < d; ++k) y += double(p[size_t(i) * d + k]) * u[k];
          acc[i] += y * y;
        }
      }
      for (int i = 0; i < d; ++i) sig[size_t(h) * d + i] = std::sqrt(acc[i] / double(ds.calib_n));
    }
  }
  if (waterfill) {
    std::vector<double> lam(d, 0.0);
    for (int h = 0; h < heads; ++h)
      for (int i = 0; i < d; ++i) lam[i] += sig[size_t(h) * d + i] * sig[size_t(h) * d + i] / heads;
    if (tq_water_fill(lam.data(), d, ds.waterfill_bits, 1, kMaxBits, cb->bits.data()) != TQ_OK)
      return TQ_EINVAL;
    cb->uniform = std::all_of(cb->bits.begin(), cb->bits.end(), [&](uint8_t b) { return b == cb->bits[0]; });
    cb->ubits = cb->uniform ? cb->bits[0] : 0;
    if (ds.layout == TQ_LAYOUT_COL && !cb->uniform) return TQ_EUNSUPPORTED;
  }

  // ----------------------------------------------------------- codebooks
  cb->cen64.assign(size_t(heads) * d * kMaxLevels, 0.0);
  cb->thr64.assign(size_t(heads) * d * (kMaxLevels - 1), 0.0);
  cb->cen32.assign(size_t(heads) * d * kMaxLevels, 0.f);
  cb->thr32.assign(size_t(heads) * d * kMaxLevels, INFINITY);
  LloydMaxResult books[kMaxBits + 1];
  bool have[kMaxBits + 1] = {};
  for (int i = 0; i < d; ++i) {
    const int b = cb->bits[i];
    if (!have[b]) {
      books[b] = ds.rotation == TQ_ROT_CALIBRATE ? lloyd_max_gaussian(b) : lloyd_max_sphere(d, b);
      have[b] = true;
    }
  }
  for (int h = 0; h < heads; ++h) {
    const double* sigma = &sig[size_t(h) * d];
    for (int i = 0; i < d; ++i) {
      const LloydMaxResult& lm = books[cb->bits[i]];
      const int L = 1 << cb->bits[i];
      for (int k = 0; k < L; ++k) {
        const double c = lm.centroids[k] * sigma[i];
        cb->cen64[(size_t(h) * d + i) * kMaxLevels + k] = c;
        cb->cen32[(size_t(h) * d + i) * kMaxLevels + k] = float(c);
      }
      for (int k = 0; k + 1 < L; ++k) {
        const double t = lm.boundaries[k] * sigma[i];
        cb->thr64[(size_t(h) * d + i) * (kMaxLevels - 1) + k] = t;
        cb->thr32[(size_t(h) * d + i) * kMaxLevels + k] = float(t);
      }
    }
  }
  // bit positions of the row-layout bit string
  cb->bitpos.assign(size_t(kMaxBits) * d, -1);
  int pos = 0;
  for (int p = 0; p < kMaxBits; ++p)
    for (int i = 0; i < d; ++i)
      if (cb->bits[i] > p) cb->bitpos[size_t(p) * d + i] = int16_t(pos++);
  fill_info(cb);
  cb->info.num_heads = heads;
  return TQ_OK;
}

tq_status build_device(tq_codebook* cb) {
  const int d = cb->desc.d;
  if (hipSetDevice(cb->device) != hipSuccess) return TQ_EDEVICE;
  const size_t nr = cb->rot32.size();
  std::vector<uint16_t> hi(nr), lo(nr);
  // fp16 hi + lo parts of 16 Pi (the factor keeps the lo parts normal); the
  // encode kernel divides it out with the per-vector scale
  for (size_t e = 0; e < nr; ++e) {
    const float v = 16.f * cb->rot32[e];
    hi[e] = f32_to_f16_rne(v);
    lo[e] = f32_to_f16_rne(v - f16_to_f32(hi[e]));
  }
  // transposed copies: query rotation reads them column-coalesced
  std::vector<float> rt(nr);
  for (size_t hh = 0; hh < nr / (size_t(d) * d); ++hh)
    for (int i = 0; i < d; ++i)
      for (int k = 0; k < d; ++k)
        rt[(hh * d + k) * d + i] = cb->rot32[(hh * d + i) * d + k];
  tq_status st;
  if ((st = upload(&cb->dev.rot, cb->rot32.data(), nr)) != TQ_OK) return st;
  if ((st = upload(&cb->dev.rot_t, rt.data(), nr)) != TQ_OK) return st;
  if ((st = upload(&cb->dev.rot_hi, hi.data(), nr)) != TQ_OK) return st;
  if ((st = upload(&cb->dev.rot_lo, lo.data(), nr)) != TQ_OK) return st;
  if (!cb->sketch32.empty()) {
    const size_t ns = cb->sketch32.size();
    std::vector<uint16_t> shi(ns), slo(ns);
    for (size_t e = 0; e < ns; ++e) {
      shi[e] = f32_to_f16_rne(cb->sketch32[e]);
      slo[e] = f32_to_f16_rne(cb->sketch32[e] - f16_to_f32(shi[e]));
    }
    const int m = cb->m;
    std::vector<float> st_(ns);
    for (int j = 0; j < m; ++j)
      for (int k = 0; k < m; ++k) st_[size_t(k) * m + j] = cb->sketch32[size_t(j) * m + k];
    if ((st = upload(&cb->dev.sketch, cb->sketch32.data(), ns)) != TQ_OK) return st;
    if ((st = upload(&cb->dev.sketch_t, st_.data(), ns)) != TQ_OK) return st;
    if ((st = upload(&cb->dev.sketch_hi, shi.data(), ns)) != TQ_OK) return st;
    if ((st = upload(&cb->dev.sketch_lo, slo.data(), ns)) != TQ_OK) return st;
  }
  if (d != 128 && d % 128 == 0 && cb->uniform && !cb->outlier) {
    // operand tiles of the wide MFMA kernels: per 128-row block and 32-column
    // tile, [hi, lo][128][32] of 16 Pi (and [128][32] of S), rows of every
    // 32-row group in the order 8a + 4h + c <- 16h + 4a + c, so that the
    // accumulator registers of a half-wave cover 16 consecutive rows
    auto perm = [](int g) { return (g & ~31) | (((g >> 2) & 1) << 4) | (((g >> 3) & 3) << 2) | (g & 3); };
    const int heads = int(nr / (size_t(d) * d)), nkt = d / 32;
    std::vector<uint16_t> rt_(nr * 2);
    for (int hh = 0; hh < heads; ++hh)
      for (int b = 0; b < d / 128; ++b)
        for (int kt = 0; kt < nkt; ++kt)
          for (int pl = 0; pl < 2; ++pl)
            for (int g = 0; g < 128; ++g)
              for (int e = 0; e < 32; ++e) {
                const size_t src = (size_t(hh) * d + size_t(b) * 128 + perm(g)) * d + size_t(kt) * 32 + e;
                const size_t dst = ((((size_t(hh) * (d / 128) + b) * nkt + kt) * 2 + pl) * 128 + g) * 32 + e;
                rt_[dst] = pl == 0 ? hi[src] : lo[src];
              }
    if ((st = upload(&cb->dev.rot_tiles, rt_.data(), rt_.size())) != TQ_OK) return st;
    if (!cb->sketch32.empty() && cb->m % 128 == 0) {
      const int m = cb->m, mkt = m / 32;
      std::vector<uint16_t> sk(size_t(m) * m);
      for (int b = 0; b < m / 128; ++b)
        for (int kt = 0; kt < mkt; ++kt)
          for (int g = 0; g < 128; ++g)
            for (int e = 0; e < 32; ++e)
              sk[((size_t(b) * mkt + kt) * 128 + g) * 32 + e] =
                  f32_to_f16_rne(cb->sketch32[(size_t(b) * 128 + perm(g)) * m + size_t(kt) * 32 + e]);
      if ((st = upload(&cb->dev.sk_tiles, sk.data(), sk.size())) != TQ_OK) return st;
    }
  }
  if ((st = upload(&cb->dev.thr, cb->thr32.data(), cb->thr32.size())) != TQ_OK) return st;
  if ((st = upload(&cb->dev.cen, cb->cen32.data(), cb->cen32.size())) != TQ_OK) return st;
  if ((st = upload(&cb->dev.bitpos, cb->bitpos.data(), cb->bitpos.size())) != TQ_OK) return st;
  if ((st = upload(&cb->dev.dim_bits, cb->bits.data(), size_t(d))) != TQ_OK) return st;
  if (!cb->hsign.empty() && d == 128) {
    std::vector<uint32_t> mask(64, 0u);
    for (int hh = 0; hh < 2; ++hh)
      for (int k = 0; k < 32; ++k) {
        const int i0 = 64 * hh + 2 * k;
        mask[hh * 32 + k] = (cb->hsign[i0] < 0 ? 0x8000u : 0u) | (cb->hsign[i0 + 1] < 0 ? 0x80000000u : 0u);
      }
    if ((st = upload(&cb->dev.had_mask, mask.data(), mask.size())) != TQ_OK) return st;
    std::vector<float> sgn(cb->hsign.begin(), cb->hsign.end());
    if ((st = upload(&cb->dev.had_sign, sgn.data(), sgn.size())) != TQ_OK) return st;
  }
  if (!cb->omask.empty())
    if ((st = upload(&cb->dev.omask, cb->omask.data(), cb->omask.size())) != TQ_OK) return st;
  if (!cb->uniform && !cb->outlier && d == 128) {
    // tail byte t -> bits 1.. of the indices of dims 0..3 (dim i at bits 5i..5i+4),
    // for the bit positions D..D+7 of the row bit string
    std::vector<uint32_t> tail(256, 0u);
    for (uint32_t t = 0; t < 256; ++t) {
      uint32_t packed = 0;
      for (int i = 0; i < 4; ++i) {
        uint32_t v = 0;
        for (int pl = 1; pl < cb->bits[i] && pl < kMaxBits; ++pl) {
          const int pos = cb->bitpos[size_t(pl) * d + i] - d;
          if (pos >= 0 && pos < 8) v |= ((t >> pos) & 1u) << pl;
        }
        packed |= (v & 31u) << (5 * i);
      }
      tail[t] = packed;
    }
    const int heads = cb->info.num_heads;
    std::vector<float> gm(size_t(heads) * 2 * d);
    for (int hh = 0; hh < heads; ++hh)
      for (int i = 0; i < d; ++i) {
        const float c0 = cb->cen32[(size_t(hh) * d + i) * kMaxLevels];
        const float c1 = cb->cen32[(size_t(hh) * d + i) * kMaxLevels + 1];
        gm[(size_t(hh) * 2 + 0) * d + i] = 0.5f * (c1 - c0);
        gm[(size_t(hh) * 2 + 1) * d + i] = 0.5f * (c1 + c0);
      }
    if ((st = upload(&cb->dev.sq_tail, tail.data(), tail.size())) != TQ_OK) return st;
    if ((st = upload(&cb->dev.sq_gm, gm.data(), gm.size())) != TQ_OK) return st;
  }
  return TQ_OK;
}

bool on_device(const tq_codebook* cb) { return cb && cb->device >= 0 && cb->dev.rot; }

tq_status map_hip(hipError_t e) {
  if (e == hipSuccess) return TQ_OK;
  if (e == hipErrorNotSupported) return TQ_EUNSUPPORTED;
  return TQ_EDEVICE;
}

int64_t decode_nsplit(int64_t max_tokens) {
  const int64_t ntiles = (max_tokens + kTile - 1) / kTile;
  return std::max<int64_t>(1, (ntiles + 7) / 8);  // <= 1024 for max_tokens <= 512K
}
constexpr int kDecodeChunkTiles = 8;

constexpr int kTopkSegments = 16;  // partial lists per key chunk of the general top-k path
// Queries per internal pass of tq_score / tq_search_topk (the grid limits of
// the d = 128 score and general top-k kernels; a multiple of the 128-query
// blocks of the wide search).  Larger query sets run as consecutive passes
// that share the workspace.
constexpr int64_t kTopkQueries = 65408;
constexpr int64_t kScoreQueries = 4 * kTopkQueries;

// Keys per chunk of the general top-k path (scores of a chunk are written to
// the workspace, then scanned): about 2^26 scores per chunk, at most 64 chunks,
// whole record tiles.
int64_t topk_chunk(int64_t nq, int64_t n) {
  int64_t c = std::max<int64_t>(4096, (int64_t(1) << 26) / std::max<int64_t>(1, nq));
  c = std::max(c, (n + 63) / 64);
  c = (c + kTile - 1) / kTile * kTile;
  return std::min(c, (n + kTile - 1) / kTile * kTile);
}

bool supported_query_d(int d) { return d % 64 == 0 && d >= 64 && d <= 4096; }

}  // namespace

CodecView tq::make_view(const tq_codebook* cb) {
  CodecView v{};
  v.d = cb->desc.d;
  v.mode = cb->desc.mode;
  v.m = cb->m;
  v.layout = cb->desc.layout;
  v.uniform = cb->uniform ? 1 : 0;
  v.ubits = cb->ubits;
  v.heads = cb->info.num_heads;
  v.code_bytes = cb->info.code_bytes;
  v.sign_bytes = cb->info.sign_bytes;
  v.tile_bytes = int(cb->info.tile_bytes);
  v.off_signs = int(cb->info.off_signs);
  v.off_nx = int(cb->info.off_nx);
  v.off_nr = int(cb->info.off_nr);
  v.tail_bits = cb->info.index_bits_total - cb->desc.d;
  v.outl = cb->outlier;
  v.o4 = cb->info.outlier_per_block;
  v.off_nxo = int(cb->info.off_nx_o);
  v.off_nro = int(cb->info.off_nr_o);
  v.split_ub_o = cb->outlier ? cb->bits[0] : 0;                // stored dim 0: outlier
  v.split_ub_r = cb->outlier ? cb->bits[cb->desc.d - 1] : 0;   // last stored dim: regular
  v.omask = cb->dev.omask;
  v.sq_ok = 0;
  if (!cb->uniform && !cb->outlier && int(cb->bits.size()) == cb->desc.d && cb->desc.d > 4) {
    bool ok = true;
    for (int i = 0; i < cb->desc.d; ++i)
      ok = ok && (i < 4 ? cb->bits[i] >= 1 && cb->bits[i] <= 5 : cb->bits[i] == 1);
    v.sq_ok = ok && cb->dev.sq_tail != nullptr;
  }
  v.rot = cb->dev.rot;
  v.rot_t = cb->dev.rot_t;
  v.rot_hi = cb->dev.rot_hi;
  v.rot_lo = cb->dev.rot_lo;
  v.sketch = cb->dev.sketch;
  v.sketch_t = cb->dev.sketch_t;
  v.sk_hi = cb->dev.sketch_hi;
  v.sk_lo = cb->dev.sketch_lo;
  v.thr = cb->dev.thr;
  v.cen = cb->dev.cen;
  v.bitpos = cb->dev.bitpos;
  v.dim_bits = cb->dev.dim_bits;
  v.sq_tail = cb->dev.sq_tail;
  v.sq_gm = cb->dev.sq_gm;
  v.had_mask = cb->dev.had_mask;
  v.had_sign = cb->dev.had_sign;
  v.rot_tiles = cb->dev.rot_tiles;
  v.sk_tiles = cb->dev.sk_tiles;
  for (int k = 0; k < kMaxLevels; ++k) {
    v.uthr[k] = cb->thr32[k];
    v.ucen[k] = cb->cen32[k];
  }
  v.qn = 0;
  v.qinvw = v.qoff = 0.f;
  if (cb->uniform && cb->ubits >= 1) {
    // bucket width: the smallest gap between boundaries over s (at least 2.5),
    // s stepped until no boundary lies within 2 % of a bucket edge; offset
    // so that every coordinate of a unit vector (|y| <= 1, plus rounding)
    // maps to a bucket >= 1, and half-integer, so that a boundary at 0 sits
    // mid-bucket
    const int nb = (1 << cb->ubits) - 1;
    double gap = 2.0;
    for (int k = 0; k + 1 < nb; ++k) gap = std::min(gap, double(cb->thr32[k + 1]) - double(cb->thr32[k]));
    for (int step = 0; step < 200 && v.qn == 0; ++step) {
      const double w = gap / (2.5 + 0.05 * step);
      const double off = std::ceil(1.05 / w) + 1.5;
      const int n = int(2.0 * off) + 2;
      if (n > kQMax) break;
      bool ok = true;
      for (int k = 0; k < nb && ok; ++k) {
        const double pos = double(cb->thr32[k]) / w + off;
        const double fr = pos - std::floor(pos);
        ok = fr >= 0.02 && fr <= 0.98;
      }
      if (ok) {
        v.qn = n;
        v.qinvw = float(1.0 / w);
        v.qoff = float(off);
      }
    }
  }
  return v;
}

namespace {

// Workspace of the wide (d != 128) query preparation, the MFMA search /
// dense scoring, and the general top-k path, laid out in this order after
// the prepared queries ([nq][d] q' and [nq][m] qs, fp32).
struct QueryWs {
  size_t qprep, wide, tiles, inv, ps, pi, scores;
  size_t total() const { return qprep + wide + tiles + inv + ps + pi + scores; }
};

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

int device_cus(int device) {
  int cus = 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

// op TQ_OP_SCORE (k = 0) or TQ_OP_TOPK
QueryWs query_ws(const tq_codebook* cb, int32_t op, int64_t nq, int64_t n, int k) {
  QueryWs w{};
  const CodecView cv = make_view(cb);
  const size_t d = size_t(cb->desc.d), m = size_t(std::max(cb->m, 1));
  w.qprep = round256(size_t(nq) * (d + m) * 4);
  if (d != 128) w.wide = round256(wide_query_prep_workspace(cv, nq));
  const bool mfma = search_mfma_supported(cv) && n < (int64_t(1) << 31);
  if (op == TQ_OP_SCORE) {
    if (d != 128) {
      const SearchPlan p = search_plan(cv, nq, n, device_cus(cb->device));
      w.tiles = p.tiles_bytes;
      w.inv = p.inv_bytes;
    }
    return w;
  }
  if (mfma) {
    const SearchPlan p = search_plan(cv, nq, n, device_cus(cb->device));
    w.tiles = p.tiles_bytes;
    w.inv = p.inv_bytes;
    w.ps = round256(size_t(nq) * p.nparts * k * 4);
    w.pi = round256(size_t(nq) * p.nparts * k * 8);
  } else {
    const int64_t chunk = topk_chunk(nq, n);
    const int64_t nchunks = (n + chunk - 1) / chunk;
    w.scores = round256(size_t(nq) * size_t(chunk) * 4);
    w.ps = round256(size_t(nq) * nchunks * kTopkSegments * k * 4);
    w.pi = round256(size_t(nq) * nchunks * kTopkSegments * k * 8);
  }
  return w;
}

}  // namespace

extern "C" {

const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported configuration";
    case TQ_EALIGN: return "misaligned pointer or stride";
    case TQ_ENOMEM: return "out of memory";
    case TQ_EWORKSPACE: return "workspace too small";
    case TQ_EDEVICE: return "HIP runtime or launch error";
  }
  return "unknown status";
}

tq_status tq_codebook_build(const tq_codebook_desc* desc, tq_codebook** out) {
  if (!desc || !out) return TQ_EINVAL;
  *out = nullptr;
  const tq_codebook_desc& ds = *desc;
  if (ds.d < 2 || ds.d > 4096) return TQ_EINVAL;
  if (ds.mode != TQ_MSE && ds.mode != TQ_PROD) return TQ_EINVAL;
  if (ds.mode == TQ_PROD && !ds.bitmap && ds.waterfill_bits <= 0 && ds.bits < 2) return TQ_EINVAL;
  if (ds.layout != TQ_LAYOUT_ROW && ds.layout != TQ_LAYOUT_COL) return TQ_EINVAL;
  if (ds.qjl_dims < 0 || ds.num_heads < 0) return TQ_EINVAL;
  if ((ds.rotation == TQ_ROT_HAAR || ds.rotation == TQ_ROT_HADAMARD) && ds.num_heads > 1 && ds.outlier_dims == 0)
    return TQ_EINVAL;
  tq_codebook* cb = new (std::nothrow) tq_codebook();
  if (!cb) return TQ_ENOMEM;
  cb->desc = ds;
  cb->device = ds.device;
  tq_status st;
  try {
    st = build_host(cb, ds);
  } catch (const std::bad_alloc&) {
    st = TQ_ENOMEM;
  }
  // the caller's host arrays are not kept
  cb->desc.bitmap = nullptr;
  cb->desc.given = nullptr;
  cb->desc.calib = nullptr;
  cb->desc.outlier_channels = nullptr;
  if (st == TQ_OK && cb->device >= 0) st = build_device(cb);
  if (st != TQ_OK) {
    free_device(cb);
    delete cb;
    return st;
  }
  *out = cb;
  return TQ_OK;
}

tq_status tq_append(const tq_codebook* cb, const void* x, int32_t x_dtype, int32_t B, int32_t H,
                    int64_t xs_b, int64_t xs_h, void* records, int64_t rs_b, int64_t rs_h,
                    const int32_t* positions, int32_t capacity, void* stream) {
  if (!cb || !x || !records || !positions) return TQ_EINVAL;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_EINVAL;
  if (B < 0 || H < 0 || capacity < 0 || xs_b < 0 || xs_h < 0 || rs_b < 0 || rs_h < 0) return TQ_EINVAL;
  if (!on_device(cb)) return TQ_EINVAL;
  if (cb->info.num_heads > 1 && cb->info.num_heads != H) return TQ_EINVAL;
  const CodecView cv = make_view(cb);
  if (!append_supported(cv)) return TQ_EUNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(records) & 3) || (rs_b & 3) || (rs_h & 3)) return TQ_EALIGN;
  if (B == 0 || H == 0 || capacity == 0) return TQ_OK;
  if (B > 65535 || H > 65535) return TQ_EUNSUPPORTED;
  if (hipSetDevice(cb->device) != hipSuccess) return TQ_EDEVICE;
  AppendArgs a{x, x_dtype == TQ_BF16, B, H, xs_b, xs_h, static_cast<uint8_t*>(records), rs_b, rs_h,
               positions, capacity, nullptr, 0, 0};
  return map_hip(launch_append(cv, a, static_cast<hipStream_t>(stream)));
}

tq_status tq_water_fill(const double* lambda, int32_t d, int32_t total_bits, int32_t min_bits,
                        int32_t max_bits, uint8_t* bits_out) {
  if (!lambda || !bits_out || d < 1) return TQ_EINVAL;
  if (min_bits < 1 || max_bits > kMaxBits || min_bits > max_bits) return TQ_EINVAL;
  if (int64_t(total_bits) < int64_t(d) * min_bits || int64_t(total_bits) > int64_t(d) * max_bits)
    return TQ_EINVAL;
  for (int i = 0; i < d; ++i)
    if (!(lambda[i] >= 0.0)) return TQ_EINVAL;
  // distortion of the b-bit Gaussian Lloyd-Max quantizer, b = min..max
  double D[kMaxBits + 1];
  for (int b = min_bits; b <= max_bits; ++b) D[b] = lloyd_max_gaussian(b).mse;
  std::vector<int> bits(d, min_bits);
  for (int64_t left = int64_t(total_bits) - int64_t(d) * min_bits; left > 0; --left) {
    int best = -1;
    double gain = -1.0;
    for (int i = 0; i < d; ++i) {
      if (bits[i] >= max_bits) continue;
      const double g = lambda[i] * (D[bits[i]] - D[bits[i] + 1]);
      if (g > gain) { gain = g; best = i; }  // strict: ties stay with the lower dim
    }
    ++bits[best];
  }
  for (int i = 0; i < d; ++i) bits_out[i] = uint8_t(bits[i]);
  return TQ_OK;
}

tq_status tq_codebook_free(tq_codebook* cb) {
  if (!cb) return TQ_EINVAL;
  if (cb->device >= 0) (void)hipSetDevice(cb->device);
  free_device(cb);
  delete cb;
  return TQ_OK;
}

tq_status tq_codebook_get_info(const tq_codebook* cb, tq_codebook_info* info) {
  if (!cb || !info) return TQ_EINVAL;
  *info = cb->info;
  return TQ_OK;
}

tq_status tq_codebook_export(const tq_codebook* cb, int32_t head, float* rot, float* sketch,
                             double* centroids, double* boundaries, int32_t* levels) {
  if (!cb) return TQ_EINVAL;
  const int d = cb->desc.d;
  if (head < 0 || head >= cb->info.num_heads) return TQ_EINVAL;
  if (rot) std::memcpy(rot, &cb->rot32[size_t(head) * d * d], sizeof(float) * d * d);
  if (sketch && !cb->sketch32.empty())
    std::memcpy(sketch, cb->sketch32.data(), sizeof(float) * cb->sketch32.size());
  if (centroids)
    std::memcpy(centroids, &cb->cen64[size_t(head) * d * kMaxLevels], sizeof(double) * d * kMaxLevels);
  if (boundaries)
    std::memcpy(boundaries, &cb->thr64[size_t(head) * d * (kMaxLevels - 1)],
                sizeof(double) * d * (kMaxLevels - 1));
  if (levels)
    for (int i = 0; i < d; ++i) levels[i] = 1 << cb->bits[i];
  return TQ_OK;
}

int64_t tq_records_bytes(const tq_codebook* cb, int64_t n) {
  if (!cb || n < 0) return -1;
  return ((n + kTile - 1) / kTile) * cb->info.tile_bytes;
}

// The argument checks of one encode (tq_encode's, short of the workspace) and
// its kernel arguments; *empty when there is nothing to encode.
static tq_status encode_check(const tq_codebook* cb, const void* x, int32_t x_dtype, int64_t batch,
                              int64_t heads, int64_t tokens, int64_t xs_b, int64_t xs_h, int64_t xs_t,
                              void* records, int64_t rs_b, int64_t rs_h, EncodeArgs* a, bool* empty) {
  *empty = false;
  if (!cb) return TQ_EINVAL;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_EINVAL;
  if (batch < 0 || heads < 0 || tokens < 0) return TQ_EINVAL;
  if (batch == 0 || heads == 0 || tokens == 0) {  // nothing to encode
    *empty = true;
    return TQ_OK;
  }
  if (!x || !records) return TQ_EINVAL;
  if (xs_b < 0 || xs_h < 0 || xs_t < cb->desc.d) return TQ_EINVAL;
  if (batch * heads > int64_t(65535) * 65535) return TQ_EUNSUPPORTED;
  if (!on_device(cb)) return TQ_EINVAL;
  if (cb->info.num_heads > 1 && heads != cb->info.num_heads) return TQ_EINVAL;
  const int d = cb->desc.d;
  if (d != 128 && (d % 128 || d > 4096 || !cb->uniform || cb->desc.layout != TQ_LAYOUT_ROW ||
                   (cb->desc.mode == TQ_PROD && cb->m != d)))
    return TQ_EUNSUPPORTED;
  const int64_t esz = x_dtype == TQ_F32 ? 4 : 2;
  if (!aligned16(x) || !aligned16(records) || (xs_t * esz) % 16 || (xs_h * esz) % 16 ||
      (xs_b * esz) % 16 || rs_b % 16 || rs_h % 16)
    return TQ_EALIGN;
  *a = EncodeArgs{x, x_dtype == TQ_BF16, batch, heads, tokens, xs_b, xs_h, xs_t,
                  static_cast<uint8_t*>(records), rs_b, rs_h};
  return TQ_OK;
}

tq_status tq_encode(const tq_codebook* cb, const void* x, int32_t x_dtype, int64_t batch,
                    int64_t heads, int64_t tokens, int64_t xs_b, int64_t xs_h, int64_t xs_t,
                    void* records, int64_t rs_b, int64_t rs_h, void* workspace,
                    size_t workspace_bytes, void* stream) {
  EncodeArgs a{};
  bool empty = false;
  const tq_status st = encode_check(cb, x, x_dtype, batch, heads, tokens, xs_b, xs_h, xs_t, records, rs_b, rs_h,
                                    &a, &empty);
  if (st != TQ_OK || empty) return st;
  const size_t need = tq_workspace_size(cb, TQ_OP_ENCODE, 0, 0, 0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return TQ_EWORKSPACE;
  if (need > 0 && !aligned16(workspace)) return TQ_EALIGN;
  if (hipSetDevice(cb->device) != hipSuccess) return TQ_EDEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cb->desc.d != 128) return map_hip(launch_encode_wide(make_view(cb), a, workspace, s));
  return map_hip(launch_encode_d128(make_view(cb), a, s));
}

tq_status tq_encode_kv(const tq_codebook* kcb, const tq_codebook* vcb, const void* k, const void* v,
                       int32_t x_dtype, int64_t batch, int64_t heads, int64_t tokens, int64_t xs_b,
                       int64_t xs_h, int64_t xs_t, void* k_records, int64_t kr_b, int64_t kr_h,
                       void* v_records, int64_t vr_b, int64_t vr_h, void* stream) {
  if (!kcb || !vcb) return TQ_EINVAL;
  EncodeArgs ka{}, va{};
  bool empty = false;
  tq_status st = encode_check(kcb, k, x_dtype, batch, heads, tokens, xs_b, xs_h, xs_t, k_records, kr_b, kr_h,
                              &ka, &empty);
  if (st != TQ_OK) return st;
  st = encode_check(vcb, v, x_dtype, batch, heads, tokens, xs_b, xs_h, xs_t, v_records, vr_b, vr_h, &va, &empty);
  if (st != TQ_OK || empty) return st;
  if (kcb->device != vcb->device) return TQ_EINVAL;
  if (kcb->desc.d != 128 || vcb->desc.d != 128) return TQ_EUNSUPPORTED;
  if (hipSetDevice(kcb->device) != hipSuccess) return TQ_EDEVICE;
  return map_hip(launch_encode_kv_d128(make_view(kcb), ka, make_view(vcb), va, static_cast<hipStream_t>(stream)));
}


size_t tq_workspace_size(const tq_codebook* cb, int32_t op, int64_t a, int64_t b, int64_t c) {
  if (!cb || a < 0 || b < 0) return 0;
  const size_t d = size_t(cb->desc.d), m = size_t(std::max(cb->m, 1));
  const size_t qprep = size_t(a) * (d + m) * 4;
  switch (op) {
    case TQ_OP_ENCODE:
      return d != 128 ? wide_encode_workspace(make_view(cb)) : 0;
    case TQ_OP_SCORE:
      return query_ws(cb, TQ_OP_SCORE, std::min(a, kScoreQueries), b, 0).total();
    case TQ_OP_DECODE: {
      if (c <= 0) return 0;
      const size_t part = size_t(a) * size_t(decode_nsplit(b)) * (2 + d) * 4;
      return round256(qprep) + round256(part);
    }
    case TQ_OP_TOPK: {
      if (c <= 0 || c > 16) return 0;
      return query_ws(cb, TQ_OP_TOPK, std::min(a, kTopkQueries), b, int(c)).total();
    }
  }
  return 0;
}

tq_status tq_score(const tq_codebook* cb, const float* q, int64_t nq, int32_t head,
                   const void* records, int64_t n, float* scores, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!cb) return TQ_EINVAL;
  if (nq < 0 || n < 0 || head < 0 || head >= cb->info.num_heads) return TQ_EINVAL;
  if (nq == 0 || n == 0) return TQ_OK;
  if (!q || !records || !scores) return TQ_EINVAL;
  if (!on_device(cb)) return TQ_EINVAL;
  if (cb->desc.layout != TQ_LAYOUT_ROW || !supported_query_d(cb->desc.d)) return TQ_EUNSUPPORTED;
  const CodecView cv = make_view(cb);
  if (cb->desc.d != 128 && (!search_mfma_supported(cv) || n >= (int64_t(1) << 31))) return TQ_EUNSUPPORTED;
  if (!aligned16(records) || !aligned16(q)) return TQ_EALIGN;
  if (nq > kScoreQueries) {
    // consecutive passes over blocks of queries (rows of q and scores)
    for (int64_t q0 = 0; q0 < nq; q0 += kScoreQueries) {
      const int64_t c = std::min(kScoreQueries, nq - q0);
      const tq_status st = tq_score(cb, q + q0 * cb->desc.d, c, head, records, n, scores + q0 * n, workspace,
                                    workspace_bytes, stream);
      if (st != TQ_OK) return st;
    }
    return TQ_OK;
  }
  const QueryWs W = query_ws(cb, TQ_OP_SCORE, nq, n, 0);
  if (!workspace || workspace_bytes < W.total()) return TQ_EWORKSPACE;
  if (!aligned16(workspace)) return TQ_EALIGN;
  if (hipSetDevice(cb->device) != hipSuccess) return TQ_EDEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  float* qr = reinterpret_cast<float*>(w);
  float* qs = qr + nq * cb->desc.d;
  if (cb->desc.d != 128) {
    tq_status st = map_hip(launch_query_prep_wide(cv, q, nq, qr, qs, w + W.qprep, s));
    if (st != TQ_OK) return st;
    const SearchPlan p = search_plan(cv, nq, n, device_cus(cb->device));
    uint8_t* t = w + W.qprep + W.wide;
    return map_hip(launch_search(cv, qr, qs, nq, static_cast<const uint8_t*>(records), n, 0, p, t,
                                 reinterpret_cast<float*>(t + W.tiles), nullptr, nullptr, nullptr, nullptr, scores,
                                 s));
  }
  QueryPrepArgs qa{q, 0, nq, 0, 1, head, qr, qs};
  tq_status st = map_hip(launch_query_prep(cv, qa, s));
  if (st != TQ_OK) return st;
  return map_hip(launch_score(cv, qr, qs, nq, static_cast<const uint8_t*>(records), n, scores, s, head));
}

}  // extern "C"

namespace {

// Checks of a paged view (see tq_kv_view): power-of-two pages, a block table
// row long enough for max_tokens, 4-byte aligned table.
tq_status check_paging(const tq_kv_view* kv, int* page_shift) {
  *page_shift = 0;
  if (!kv->block_table) return TQ_OK;
  const int pt = kv->page_tiles;
  if (pt < 1 || (pt & (pt - 1)) || pt > (1 << 20)) return TQ_EINVAL;
  while ((1 << *page_shift) < pt) ++*page_shift;
  const int64_t ntiles = (int64_t(kv->max_tokens) + kTile - 1) / kTile;
  if (int64_t(kv->max_pages) * pt < ntiles) return TQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(kv->block_table) & 3) return TQ_EALIGN;
  return TQ_OK;
}

// Decode attention over seq_lens[b] + len_add tokens (see tq_decode_attend).
tq_status decode_impl(const tq_codebook* kcb, const tq_codebook* vcb, const void* q, int32_t q_dtype,
                      int32_t B, int32_t Hq, int32_t Hkv, const tq_kv_view* kv, float softmax_scale,
                      float* out, void* workspace, size_t workspace_bytes, void* stream, int len_add,
                      bool checks_only) {
  if (!kcb || !vcb || !q || !kv || !out || !kv->k_records || !kv->v_records) return TQ_EINVAL;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_EINVAL;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || kv->max_tokens < 0) return TQ_EINVAL;
  if (!on_device(kcb) || !on_device(vcb) || kcb->device != vcb->device) return TQ_EINVAL;
  if (kcb->desc.d != 128 || vcb->desc.d != 128) return TQ_EUNSUPPORTED;
  // values: mse, as COL records of a uniform codec with up to 4 index bits
  // or of the 2.5-bit split (MFMA kernel only), or as ROW records of a
  // uniform or an outlier-channel split codec
  if (kcb->desc.layout != TQ_LAYOUT_ROW || vcb->desc.mode != TQ_MSE) return TQ_EUNSUPPORTED;
  if (vcb->desc.layout == TQ_LAYOUT_COL ? (!vcb->uniform || vcb->ubits > 4) && vcb->outlier == 0
                                        : !(vcb->uniform || vcb->outlier > 0))
    return TQ_EUNSUPPORTED;
  if (vcb->desc.layout == TQ_LAYOUT_COL && vcb->outlier > 0 &&
      !decode_mfma_supported(make_view(kcb), make_view(vcb), Hq / Hkv))
    return TQ_EUNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return TQ_EUNSUPPORTED;
  if (kcb->info.num_heads > 1 && kcb->info.num_heads != Hkv) return TQ_EINVAL;
  if (vcb->info.num_heads > 1 && vcb->info.num_heads != Hkv) return TQ_EINVAL;
  if (kcb->desc.mode == TQ_PROD && kcb->m != 128 && kcb->m > 8) return TQ_EUNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return TQ_EINVAL;
  if (!aligned16(kv->k_records) || !aligned16(kv->v_records) || kv->k_stride_seq % 16 ||
      kv->k_stride_head % 16 || kv->v_stride_seq % 16 || kv->v_stride_head % 16 || !aligned16(q))
    return TQ_EALIGN;
  int page_shift = 0;
  if (const tq_status ps = check_paging(kv, &page_shift); ps != TQ_OK) return ps;
  if (B == 0) return TQ_OK;
  if (B > 65535 || decode_nsplit(kv->max_tokens) > 1024) return TQ_EUNSUPPORTED;
  if (kv->max_tokens == 0) {
    // an empty cache: every output is zero, no record or workspace is touched
    if (checks_only) return TQ_OK;
    if (hipSetDevice(kcb->device) != hipSuccess) return TQ_EDEVICE;
    return map_hip(launch_fill_zero(out, int64_t(B) * Hq * 128, static_cast<hipStream_t>(stream)));
  }
  const int64_t nqt = int64_t(B) * Hq;
  if (!workspace || workspace_bytes < tq_workspace_size(kcb, TQ_OP_DECODE, nqt, kv->max_tokens, Hkv))
    return TQ_EWORKSPACE;
  if (!aligned16(workspace)) return TQ_EALIGN;
  if (checks_only) return TQ_OK;
  if (hipSetDevice(kcb->device) != hipSuccess) return TQ_EDEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const CodecView kc = make_view(kcb), vc = make_view(vcb);
  const size_t d = 128, m = size_t(std::max(kcb->m, 1));
  float* qr = static_cast<float*>(workspace);
  float* qs = qr + nqt * d;
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                         ((size_t(nqt) * (d + m) * 4 + 255) & ~size_t(255)));
  // the MFMA decode rotates its queries itself; the general path reads them
  // prepared
  if (!decode_mfma_supported(kc, vc, G)) {
    QueryPrepArgs qa{q, q_dtype == TQ_BF16, nqt, G, Hkv, 0, qr, qs};
    const tq_status st = map_hip(launch_query_prep(kc, qa, s));
    if (st != TQ_OK) return st;
  }
  DecodeArgs da{};
  da.qr = qr;
  da.qs = qs;
  da.q = q;
  da.q_bf16 = q_dtype == TQ_BF16;
  da.B = B;
  da.Hq = Hq;
  da.Hkv = Hkv;
  da.krec = static_cast<const uint8_t*>(kv->k_records);
  da.vrec = static_cast<const uint8_t*>(kv->v_records);
  da.ks_seq = kv->k_stride_seq;
  da.ks_head = kv->k_stride_head;
  da.vs_seq = kv->v_stride_seq;
  da.vs_head = kv->v_stride_head;
  da.max_tokens = kv->max_tokens;
  da.seq_lens = kv->seq_lens;
  da.scale = softmax_scale;
  da.len_add = len_add;
  da.block_table = kv->block_table;
  da.page_shift = page_shift;
  da.max_pages = kv->max_pages;
  // splits of 8 tiles, widened while the grid still fills every resident
  // workgroup slot (two per CU): fewer block set-ups and partials for large
  // batches, down to one split per sequence (then no merge pass at all);
  // never more splits than the workspace holds.  With fewer (sequence, KV
  // head) pairs than CUs the MFMA kernel runs 8-wave workgroups, one per CU,
  // on splits of 16 tiles (two per wave, as with 8 tiles over 4 waves), so
  // that each CU sets up once
  {
    const int64_t ntiles = (int64_t(kv->max_tokens) + kTile - 1) / kTile;
    int cus = 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, kcb->device) != hipSuccess) cus = 256;
    const bool wide = int64_t(B) * Hkv < cus && decode_mfma_supported(kc, vc, Hq / Hkv);
    const int64_t slots = (wide ? 1 : 2) * int64_t(cus);
    int chunk = wide ? 2 * kDecodeChunkTiles : kDecodeChunkTiles;
    while (chunk < 1024 && chunk < ntiles &&
           int64_t(B) * Hkv * ((ntiles + 2 * chunk - 1) / (2 * chunk)) >= slots)
      chunk *= 2;
    da.chunk_tiles = chunk;
    da.nsplit = int(std::max<int64_t>(1, (ntiles + chunk - 1) / chunk));
    da.waves = wide && da.nsplit > 1 ? 8 : 4;
  }
  da.part = part;
  da.out = out;
  return map_hip(launch_decode(kc, vc, da, s));
}

}  // namespace

tq_status tq::decode_attend_ws(const tq_codebook* kcb, const tq_codebook* vcb, const void* q, int32_t q_dtype,
                               int32_t B, int32_t Hq, int32_t Hkv, const tq_kv_view* kv, float softmax_scale,
                               float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kcb, vcb, q, q_dtype, B, Hq, Hkv, kv, softmax_scale, out, workspace, workspace_bytes,
                     stream, 0, false);
}

extern "C" {

tq_status tq_decode_attend(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                           int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                           const tq_kv_view* kv, float softmax_scale, float* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kcb, vcb, q, q_dtype, B, Hq, Hkv, kv, softmax_scale, out, workspace, workspace_bytes,
                     stream, 0, false);
}

tq_status tq_decode_step(const tq_codebook* kcb, const tq_codebook* vcb, const void* q,
                         int32_t q_dtype, const void* k_new, const void* v_new, int32_t new_dtype,
                         int32_t B, int32_t Hq, int32_t Hkv, const tq_kv_view* kv,
                         float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!kv || !kv->seq_lens || !k_new || !v_new) return TQ_EINVAL;
  if (new_dtype != TQ_F32 && new_dtype != TQ_BF16) return TQ_EINVAL;
  // every check of both parts runs before anything is launched
  tq_status st = decode_impl(kcb, vcb, q, q_dtype, B, Hq, Hkv, kv, softmax_scale, out, workspace,
                             workspace_bytes, stream, 1, true);
  if (st != TQ_OK || B == 0) return st;
  if (kv->max_tokens == 0)  // no slot to append to: the attention over nothing is zero
    return decode_impl(kcb, vcb, q, q_dtype, B, Hq, Hkv, kv, softmax_scale, out, workspace, workspace_bytes,
                       stream, 1, false);
  if (kcb->info.num_heads > 1 && kcb->info.num_heads != Hkv) return TQ_EINVAL;
  const CodecView kc = make_view(kcb), vc = make_view(vcb);
  if (!append_supported(kc) || !append_supported(vc)) return TQ_EUNSUPPORTED;
  if ((kv->k_stride_seq & 3) || (kv->k_stride_head & 3) || (kv->v_stride_seq & 3) || (kv->v_stride_head & 3))
    return TQ_EALIGN;
  if (B > 65535 || Hkv > 65535) return TQ_EUNSUPPORTED;
  int page_shift = 0;
  check_paging(kv, &page_shift);
  if (hipSetDevice(kcb->device) != hipSuccess) return TQ_EDEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t d = kcb->desc.d;
  // the new tokens go to slot seq_lens[b]; slots at or past max_tokens are skipped
  AppendArgs ka{k_new, new_dtype == TQ_BF16, B, Hkv, Hkv * d, d,
                static_cast<uint8_t*>(const_cast<void*>(kv->k_records)), kv->k_stride_seq, kv->k_stride_head,
                kv->seq_lens, kv->max_tokens, kv->block_table, page_shift, kv->max_pages};
  AppendArgs va = ka;
  va.x = v_new;
  va.rec = static_cast<uint8_t*>(const_cast<void*>(kv->v_records));
  va.rs_b = kv->v_stride_seq;
  va.rs_h = kv->v_stride_head;
  if ((st = map_hip(launch_append_pair(kc, ka, vc, va, s))) != TQ_OK) return st;
  return decode_impl(kcb, vcb, q, q_dtype, B, Hq, Hkv, kv, softmax_scale, out, workspace, workspace_bytes,
                     stream, 1, false);
}

tq_status tq_search_topk(const tq_codebook* cb, const float* q, int64_t nq,
                         const void* records, int64_t n, int32_t k, float* top_scores,
                         int64_t* top_ids, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!cb || !q || !records || !top_scores || !top_ids) return TQ_EINVAL;
  if (nq < 0 || n < 0 || k < 1) return TQ_EINVAL;
  if (k > 16) return TQ_EUNSUPPORTED;
  if (!on_device(cb)) return TQ_EINVAL;
  if (cb->desc.layout != TQ_LAYOUT_ROW || !supported_query_d(cb->desc.d) || cb->info.num_heads != 1)
    return TQ_EUNSUPPORTED;
  const CodecView cv = make_view(cb);
  const bool mfma = search_mfma_supported(cv) && n < (int64_t(1) << 31);
  if (cb->desc.d != 128 && !mfma) return TQ_EUNSUPPORTED;
  if (!aligned16(records) || !aligned16(q)) return TQ_EALIGN;
  if (nq == 0) return TQ_OK;
  if (n < k) return TQ_EINVAL;
  if (nq > kTopkQueries) {
    // consecutive passes over blocks of queries (rows of q and of the lists)
    for (int64_t q0 = 0; q0 < nq; q0 += kTopkQueries) {
      const int64_t c = std::min(kTopkQueries, nq - q0);
      const tq_status st = tq_search_topk(cb, q + q0 * cb->desc.d, c, records, n, k, top_scores + q0 * k,
                                          top_ids + q0 * k, workspace, workspace_bytes, stream);
      if (st != TQ_OK) return st;
    }
    return TQ_OK;
  }
  const QueryWs W = query_ws(cb, TQ_OP_TOPK, nq, n, k);
  if (!workspace || workspace_bytes < W.total()) return TQ_EWORKSPACE;
  if (!aligned16(workspace)) return TQ_EALIGN;
  if (hipSetDevice(cb->device) != hipSuccess) return TQ_EDEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t d = size_t(cb->desc.d);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  float* qr = reinterpret_cast<float*>(w);
  float* qs = qr + nq * d;
  uint8_t* tiles = w + W.qprep + W.wide;
  float* inv = reinterpret_cast<float*>(tiles + W.tiles);
  float* pss = reinterpret_cast<float*>(tiles + W.tiles + W.inv);
  int64_t* psi = reinterpret_cast<int64_t*>(tiles + W.tiles + W.inv + W.ps);
  float* sc = reinterpret_cast<float*>(tiles + W.tiles + W.inv + W.ps + W.pi);
  tq_status st;
  if (cb->desc.d != 128) {
    st = map_hip(launch_query_prep_wide(cv, q, nq, qr, qs, w + W.qprep, s));
  } else {
    QueryPrepArgs qa{q, 0, nq, 0, 1, 0, qr, qs};
    st = map_hip(launch_query_prep(cv, qa, s));
  }
  if (st != TQ_OK) return st;
  const uint8_t* rec = static_cast<const uint8_t*>(records);
  if (mfma) {
    const SearchPlan p = search_plan(cv, nq, n, device_cus(cb->device));
    return map_hip(launch_search(cv, qr, qs, nq, rec, n, k, p, tiles, inv, pss, psi, top_scores, top_ids, nullptr,
                                 s));
  }
  // general codecs (d = 128): scores of one key chunk at a time in the
  // workspace, each chunk scanned into 16 partial lists, then one merge
  const int64_t chunk = topk_chunk(nq, n);
  const int64_t nchunks = (n + chunk - 1) / chunk;
  const int total = int(nchunks * kTopkSegments);
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t r0 = c * chunk, rows = std::min(chunk, n - r0);
    hipError_t e = launch_score(cv, qr, qs, nq, rec + (r0 / kTile) * cv.tile_bytes, rows, sc, s);
    if (e != hipSuccess) return map_hip(e);
    e = launch_topk_segments(sc, rows, rows, r0, nq, k, kTopkSegments, int(c) * kTopkSegments, total, pss, psi, s);
    if (e != hipSuccess) return map_hip(e);
  }
  return map_hip(launch_topk_merge(pss, psi, nq, total, k, top_scores, top_ids, s));
}

}  // extern "C"
