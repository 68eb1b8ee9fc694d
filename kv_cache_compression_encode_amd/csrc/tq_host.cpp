// Host-side mathematics of the codec builder: the counter-based generator of
// Pi and S, Householder QR, Lloyd-Max by Gauss-Legendre quadrature and the
// Jacobi eigensolver used for SpectralQuant calibration.  Runs once per
// codebook ("solved once, offline": TurboQuant paper review, "Method").
#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>

#include "tq_internal.h"

namespace tq {

namespace {
// Run f(j) for j in [lo, hi) on up to 16 host threads (large ranges only).
template <class F>
void parallel_for(int lo, int hi, F f) {
  const int n = hi - lo;
  int nt = int(std::min(16u, std::max(1u, std::thread::hardware_concurrency())));
  if (n < 256) nt = 1;
  if (nt <= 1) {
    for (int j = lo; j < hi; ++j) f(j);
    return;
  }
  std::vector<std::thread> th;
  const int per = (n + nt - 1) / nt;
  for (int t = 0; t < nt; ++t) {
    const int a = lo + t * per, b = std::min(hi, a + per);
    if (a >= b) break;
    th.emplace_back([=] { for (int j = a; j < b; ++j) f(j); });
  }
  for (auto& x : th) x.join();
}
}  // namespace

// ------------------------------------------------------------------ Philox
// Philox4x32-10 as defined by Salmon, Moraes, Dror and Shaw (SC'11): ten
// rounds of two 32x32->64-bit multiplies with a Weyl-sequence key schedule.
void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = uint64_t(0xD2511F53u) * c[0];
    const uint64_t p1 = uint64_t(0xCD9E8D57u) * c[2];
    const uint32_t n0 = uint32_t(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n1 = uint32_t(p1);
    const uint32_t n2 = uint32_t(p0 >> 32) ^ c[3] ^ k1;
    const uint32_t n3 = uint32_t(p0);
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
  }
  std::memcpy(out, c, sizeof(c));
}

// Block i of stream s under seed: counter (i lo, i hi, s, 0), key (seed lo,
// seed hi); its words (w0, w1) and (w2, w3) each give two normals by
// Box-Muller with uniforms (w + 1/2) 2^-32.
void philox_normals(uint64_t seed, uint32_t stream, int64_t count, double* out) {
  const uint32_t key[2] = {uint32_t(seed), uint32_t(seed >> 32)};
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t blk = 0; blk * 4 < count; ++blk) {
    const uint32_t ctr[4] = {uint32_t(blk), uint32_t(uint64_t(blk) >> 32), stream, 0u};
    uint32_t w[4];
    philox4x32_10(ctr, key, w);
    double v[4];
    for (int pair = 0; pair < 2; ++pair) {
      const double u1 = (double(w[2 * pair]) + 0.5) * 0x1p-32;
      const double u2 = (double(w[2 * pair + 1]) + 0.5) * 0x1p-32;
      const double rho = std::sqrt(-2.0 * std::log(u1));
      v[2 * pair] = rho * std::cos(two_pi * u2);
      v[2 * pair + 1] = rho * std::sin(two_pi * u2);
    }
    for (int j = 0; j < 4 && blk * 4 + j < count; ++j) out[blk * 4 + j] = v[j];
  }
}

// ---------------------------------------------------------- Householder QR
// Column-major working copy; reflector k zeroes column k below the diagonal.
void haar_from_gaussian(int n, const double* g, double* pi) {
  std::vector<double> a(size_t(n) * n);  // column-major: a[j*n + i] = g[i][j]
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) a[size_t(j) * n + i] = g[size_t(i) * n + j];
  std::vector<double> vs(size_t(n) * n, 0.0);  // reflector k in vs[k*n + k ..]
  std::vector<double> rdiag(n);
  for (int k = 0; k < n; ++k) {
    double* col = &a[size_t(k) * n];
    double norm2 = 0;
    for (int i = k; i < n; ++i) norm2 += col[i] * col[i];
    const double norm = std::sqrt(norm2);
    const double alpha = col[k] >= 0 ? -norm : norm;
    double* v = &vs[size_t(k) * n];
    for (int i = k; i < n; ++i) v[i] = col[i];
    v[k] -= alpha;
    double vn2 = 0;
    for (int i = k; i < n; ++i) vn2 += v[i] * v[i];
    rdiag[k] = alpha;
    if (vn2 == 0) continue;
    const double inv = 1.0 / std::sqrt(vn2);
    for (int i = k; i < n; ++i) v[i] *= inv;
    parallel_for(k, n, [&](int j) {
      double* cj = &a[size_t(j) * n];
      double dot = 0;
      for (int i = k; i < n; ++i) dot += v[i] * cj[i];
      dot *= 2;
      for (int i = k; i < n; ++i) cj[i] -= dot * v[i];
    });
  }
  // Q = H_0 H_1 ... H_{n-1} applied to the identity, column by column.
  std::vector<double> q(size_t(n) * n, 0.0);  // column-major
  for (int j = 0; j < n; ++j) q[size_t(j) * n + j] = 1.0;
  for (int k = n - 1; k >= 0; --k) {
    const double* v = &vs[size_t(k) * n];
    parallel_for(0, n, [&](int j) {
      double* qj = &q[size_t(j) * n];
      double dot = 0;
      for (int i = k; i < n; ++i) dot += v[i] * qj[i];
      dot *= 2;
      for (int i = k; i < n; ++i) qj[i] -= dot * v[i];
    });
  }
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      const double s = rdiag[j] < 0 ? -1.0 : 1.0;
      pi[size_t(i) * n + j] = q[size_t(j) * n + i] * s;
    }
}

// ------------------------------------------------------------- Lloyd-Max
namespace {

// 16-point Gauss-Legendre nodes/weights on [-1, 1] (positive half), computed
// once by Newton iteration on the Legendre polynomial.
struct GaussLegendre16 {
  double x[16], w[16];
  GaussLegendre16() {
    const int n = 16;
    for (int i = 0; i < n / 2; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      double dp = 1;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1, p1 = 0;
        for (int j = 1; j <= n; ++j) {
          const double p2 = p1;
          p1 = p0;
          p0 = ((2.0 * j - 1) * z * p1 - (j - 1.0) * p2) / j;
        }
        dp = n * (z * p0 - p1) / (z * z - 1);
        const double dz = p0 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-15) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1 - z * z) * dp * dp);
      x[n - 1 - i] = -z;
      w[n - 1 - i] = w[i];
    }
  }
};
const GaussLegendre16& gl16() {
  static GaussLegendre16 g;
  return g;
}

// Integrals of (1, t) against an (unnormalised) density over [a, b], by
// composite 16-point Gauss-Legendre with panels no wider than `panel`.
template <class Density, class Coord>
void cell_integrals(double a, double b, double panel, Density dens, Coord coord,
                    double* m0, double* m1) {
  *m0 = *m1 = 0;
  if (!(b > a)) return;
  const int np = std::max(2, int(std::ceil((b - a) / panel)));
  const double h = (b - a) / np;
  const auto& g = gl16();
  for (int p = 0; p < np; ++p) {
    const double c = a + (p + 0.5) * h;
    for (int k = 0; k < 16; ++k) {
      const double s = c + 0.5 * h * g.x[k];
      const double w = 0.5 * h * g.w[k] * dens(s);
      *m0 += w;
      *m1 += w * coord(s);
    }
  }
}

// Lloyd's iteration on a symmetric law given by cell integrals over a
// parameter range [lo, hi] (t = coord(s)).  Same stopping rule as used
// throughout: largest centroid move below 1e-16 max|c| or no new minimum of
// the move for 500 steps.
template <class Cells>
LloydMaxResult lloyd(int bits, double init_spread, Cells cells) {
  const int L = 1 << bits;
  std::vector<double> c(L), t(L - 1), nc(L);
  for (int k = 0; k < L; ++k) c[k] = init_spread * (-1.0 + (2.0 * k + 1.0) / L);
  double best = std::numeric_limits<double>::infinity();
  int best_it = 0, it = 0;
  for (it = 1; it <= 200000; ++it) {
    for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    double delta = 0, cmax = 0;
    for (int k = 0; k < L; ++k) {
      double m0, m1;
      cells(k == 0 ? -INFINITY : t[k - 1], k == L - 1 ? INFINITY : t[k], &m0, &m1);
      nc[k] = m1 / m0;
      delta = std::max(delta, std::fabs(nc[k] - c[k]));
      cmax = std::max(cmax, std::fabs(nc[k]));
    }
    c.swap(nc);
    if (delta < best) { best = delta; best_it = it; }
    if (delta < 1e-16 * cmax || it - best_it > 500) break;
  }
  std::vector<double> s(L);
  for (int k = 0; k < L; ++k) s[k] = 0.5 * (c[k] - c[L - 1 - k]);
  LloydMaxResult r;
  r.centroids = s;
  r.boundaries.resize(L - 1);
  for (int k = 0; k + 1 < L; ++k) r.boundaries[k] = 0.5 * (s[k] + s[k + 1]);
  if (L % 2 == 0) r.boundaries[L / 2 - 1] = 0.0;
  r.iterations = it;
  return r;
}

}  // namespace

// Coordinate of a uniform unit vector in R^d: density proportional to
// (1 - t^2)^((d-3)/2) on [-1, 1].  With t = sin(theta) the integrand becomes
// cos(theta)^(d-2) d(theta), smooth on the whole range, so the quadrature is
// done in theta.
LloydMaxResult lloyd_max_sphere(int d, int bits) {
  const double sig = 1.0 / std::sqrt(double(d));
  const double half_pi = 0.5 * M_PI;
  const double lim = std::min(half_pi, 14.0 * sig);  // mass beyond ~e^-98
  const double panel = std::min(0.25, 0.5 * sig);
  auto dens = [d](double th) { return std::pow(std::cos(th), d - 2); };
  auto coord = [](double th) { return std::sin(th); };
  double z0, z1;
  cell_integrals(-lim, lim, panel, dens, coord, &z0, &z1);
  auto cells = [&](double a, double b, double* m0, double* m1) {
    const double ta = std::isinf(a) ? -lim : std::max(-lim, std::asin(std::max(-1.0, a)));
    const double tb = std::isinf(b) ? lim : std::min(lim, std::asin(std::min(1.0, b)));
    cell_integrals(ta, tb, panel, dens, coord, m0, m1);
    *m0 /= z0;
    *m1 /= z0;
  };
  LloydMaxResult r = lloyd(bits, 2.5 * sig, cells);
  // per-coordinate mse = E[T^2] - sum_k c_k M1_k at the centroid condition,
  // recomputed here directly as sum_k int (t - c_k)^2 f.
  double mse = 0;
  const int L = 1 << bits;
  for (int k = 0; k < L; ++k) {
    const double a = k == 0 ? -INFINITY : r.boundaries[k - 1];
    const double b = k == L - 1 ? INFINITY : r.boundaries[k];
    const double ta = std::isinf(a) ? -lim : std::asin(a);
    const double tb = std::isinf(b) ? lim : std::asin(b);
    const double ck = r.centroids[k];
    double m0, m1;
    cell_integrals(ta, tb, panel, dens,
                   [ck](double th) { const double e = std::sin(th) - ck; return e * e; }, &m0, &m1);
    mse += m1 / z0;
  }
  r.mse = mse;
  return r;
}

LloydMaxResult lloyd_max_gaussian(int bits) {
  const double lim = 14.0;
  auto dens = [](double t) { return std::exp(-0.5 * t * t); };
  auto coord = [](double t) { return t; };
  double z0, z1;
  cell_integrals(-lim, lim, 0.25, dens, coord, &z0, &z1);
  auto cells = [&](double a, double b, double* m0, double* m1) {
    const double ta = std::isinf(a) ? -lim : std::max(-lim, a);
    const double tb = std::isinf(b) ? lim : std::min(lim, b);
    cell_integrals(ta, tb, 0.25, dens, coord, m0, m1);
    *m0 /= z0;
    *m1 /= z0;
  };
  LloydMaxResult r = lloyd(bits, 2.5, cells);
  double mse = 0;
  const int L = 1 << bits;
  for (int k = 0; k < L; ++k) {
    const double ta = k == 0 ? -lim : r.boundaries[k - 1];
    const double tb = k == L - 1 ? lim : r.boundaries[k];
    const double ck = r.centroids[k];
    double m0, m1;
    cell_integrals(ta, tb, 0.25, dens, [ck](double t) { return (t - ck) * (t - ck); }, &m0, &m1);
    mse += m1 / z0;
  }
  r.mse = mse;
  return r;
}

// ------------------------------------------------------------------ Jacobi
void symmetric_eigen(int n, const double* a_in, double* lambda, double* rows) {
  std::vector<double> a(a_in, a_in + size_t(n) * n);
  std::vector<double> v(size_t(n) * n, 0.0);  // columns = eigenvectors
  for (int i = 0; i < n; ++i) v[size_t(i) * n + i] = 1.0;
  auto A = [&](int i, int j) -> double& { return a[size_t(i) * n + j]; };
  double total = 0;
  for (double x : a) total += x * x;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0;
    for (int i = 0; i < n; ++i)
      for (int j = i + 1; j < n; ++j) off += A(i, j) * A(i, j);
    if (off <= 1e-30 * total) break;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) {
        const double apq = A(p, q);
        if (std::fabs(apq) < 1e-300) continue;
        const double theta = (A(q, q) - A(p, p)) / (2 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1));
        const double c = 1 / std::sqrt(t * t + 1), s = t * c;
        for (int k = 0; k < n; ++k) {  // columns p, q
          const double akp = A(k, p), akq = A(k, q);
          A(k, p) = c * akp - s * akq;
          A(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) {  // rows p, q
          const double apk = A(p, k), aqk = A(q, k);
          A(p, k) = c * apk - s * aqk;
          A(q, k) = s * apk + c * aqk;
        }
        for (int k = 0; k < n; ++k) {
          const double vkp = v[size_t(k) * n + p], vkq = v[size_t(k) * n + q];
          v[size_t(k) * n + p] = c * vkp - s * vkq;
          v[size_t(k) * n + q] = s * vkp + c * vkq;
        }
      }
  }
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return A(x, x) > A(y, y); });
  for (int r = 0; r < n; ++r) {
    const int col = order[r];
    lambda[r] = A(col, col);
    int arg = 0;
    double best = -1;
    for (int k = 0; k < n; ++k) {
      const double m = std::fabs(v[size_t(k) * n + col]);
      if (m > best) { best = m; arg = k; }
    }
    const double s = v[size_t(arg) * n + col] < 0 ? -1.0 : 1.0;
    for (int k = 0; k < n; ++k) rows[size_t(r) * n + k] = s * v[size_t(k) * n + col];
  }
}

uint16_t f32_to_bf16_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return uint16_t((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return uint16_t(u >> 16);
}

// IEEE binary16 with round-to-nearest-even (finite inputs; overflow -> inf).
uint16_t f32_to_f16_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x7f800000u) return uint16_t(sign | 0x7c00u | (a > 0x7f800000u ? 0x200u : 0));
  const int e = int(a >> 23) - 127;
  if (e > 15) return uint16_t(sign | 0x7c00u);
  uint32_t mant = (a & 0x7fffffu) | 0x800000u;  // 24-bit significand
  int shift;                                     // bits dropped from the 24-bit significand
  uint32_t expo;
  if (e >= -14) { shift = 13; expo = uint32_t(e + 15); }
  else { shift = 13 + (-14 - e); expo = 0; if (shift > 24) return uint16_t(sign); }
  const uint32_t keep = mant >> shift, rest = mant & ((1u << shift) - 1), half = 1u << (shift - 1);
  uint32_t r = keep + ((rest > half || (rest == half && (keep & 1))) ? 1 : 0);
  uint32_t bits;
  if (expo == 0) bits = r;                                   // subnormal (r may carry into normal)
  else bits = (expo << 10) + (r - 0x400u);                   // r in [0x400, 0x800]
  return uint16_t(sign | bits);
}

float f16_to_f32(uint16_t h) {
  const uint32_t sign = uint32_t(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1f, m = h & 0x3ff;
  float v;
  if (e == 0) v = std::ldexp(float(m), -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(float(m | 0x400u), int(e) - 25);
  uint32_t u;
  std::memcpy(&u, &v, 4);
  u |= sign;
  std::memcpy(&v, &u, 4);
  return v;
}

float bf16_to_f32(uint16_t h) {
  const uint32_t u = uint32_t(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace tq
