"""Plain CPU oracle of the TurboQuant / SpectralQuant codec (fp64).

Its rotations, sketches, scores and quantizer are plain loops in C
(tq_loops.c, built with gcc by build_loops.py and loaded through ctypes);
the rest is numpy, with library routines only for the QR and eigensolves
that construct Pi.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
``cpu_baseline`` leg use it.  It shares no code, tables or constants with the
HIP library; the two meet only through the seeded input generators in
``synth`` and through the record layout, which both implement from its
written specification.

What it computes, step by step, and where the pages define it:

* Random rotation Pi (seeded Haar orthogonal, QR of a Gaussian matrix) and the
  Gaussian sketch S -- TurboQuant paper review, "Method"; the launch kit names
  the dense-QR rotation mode (OnlyTerp/turboquant LAUNCH.md, Show HN post).
  Its other mode, a randomized Hadamard rotation H diag(s) / sqrt(d) (same
  launch post: the O(d log d) mode, "random Hadamard rotation").
* Lloyd-Max scalar codebook for the post-rotation coordinate law (a Beta law,
  about N(0, 1/d)) -- paper review, "Method" and the summary under the title.
* TurboQuant-mse: store ||x||, rotate x/||x||, quantize every coordinate to the
  nearest centroid -- paper review, "Method" and "Limitations" (norms stored
  separately).
* TurboQuant-prod: b-1 bits of mse codes, then a 1-bit QJL sketch sign(S r) of
  the residual r with the unbiased estimator
  ||r|| sqrt(pi/2)/m <S q', sign(S r)> -- paper review, "Method", "Key idea",
  "Results" (exactly unbiased); the news article on the KV-cache debate calls
  the residual stage a one-bit Johnson-Lindenstrauss transform.
* SpectralQuant: eigenbasis of the calibrated key covariance as the rotation,
  water-filled bits on the top dims, QJL signs on the 4 signal dims only --
  SpectralQuant thread, tweets 4, 5 and 6.
* Scoring, decode attention (softmax(q.k / sqrt(d)) . v over the compressed
  cache) and top-k search -- paper review, "Background", "Validation" and the
  "Sparks" list (rotation and codebook lookup fused into attention).

Readings where the pages are silent (each listed with the design notes):
the generator of Pi and S (Philox4x32-10 + Box-Muller, below); the Hadamard
mode's construction (one sign layer s, then Sylvester H, scaled by 1/sqrt(d);
s from bit 0 of the sign stream's words); S stored in
fp16 (the draws rounded to fp32, then fp16); fp16 norms;
ties go to the upper cell; sign(0) = +1; the sketch acts on the rotated
residual, so the query sketch is S (Pi q); the record layout of the library.

The codec's parameters (Pi, S, centroids, boundaries) are stored in fp32 by
the library, so the oracle evaluates with the fp32-rounded parameters in fp64
arithmetic.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
from scipy import special

# ---------------------------------------------------------------------------
# Plain loops (tq_loops.c): the rotations, sketches, scores and the quantizer
# below run as textbook fp64 loops, one dot product or one count per output
# in index order, built with gcc by build_loops.py.
# ---------------------------------------------------------------------------
_LOOPS = None


def _loops():
    global _LOOPS
    if _LOOPS is None:
        from oracle import build_loops
        lib = ctypes.CDLL(build_loops.build())
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.tq_oracle_matmul_nt.argtypes = [dp, dp, dp, i64, i64, i64]
        lib.tq_oracle_matmul_nt.restype = None
        lib.tq_oracle_count_le.argtypes = [dp, i64, dp, i64, i64, lp, i64]
        lib.tq_oracle_count_le.restype = None
        _LOOPS = lib
    return _LOOPS


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def dot_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """c[i][j] = sum_t a[i][t] b[j][t] (every row of a against every row of b), by plain loops."""
    a = np.ascontiguousarray(np.atleast_2d(a), dtype=np.float64)
    b = np.ascontiguousarray(np.atleast_2d(b), dtype=np.float64)
    if a.shape[1] != b.shape[1]:
        raise ValueError("rows of different lengths")
    c = np.empty((a.shape[0], b.shape[0]))
    if c.size:
        _loops().tq_oracle_matmul_nt(_dptr(a), _dptr(b), _dptr(c), a.shape[0], b.shape[0], a.shape[1])
    return c


def count_le(t: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Number of entries of t that are <= y, for every element of the 1-D array y."""
    t = np.ascontiguousarray(t, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape[0], dtype=np.int64)
    if y.size:
        _loops().tq_oracle_count_le(_dptr(t), t.shape[0], _dptr(y), y.shape[0], 1,
                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1)
    return out

# ---------------------------------------------------------------------------
# Counter-based generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
# "Parallel random numbers: as easy as 1, 2, 3", SC'11).  Written here from
# that published definition; the library carries its own implementation.
# ---------------------------------------------------------------------------
_MASK32 = np.uint64(0xFFFFFFFF)
_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = np.uint64(0x9E3779B9)
_PHILOX_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds.  counter: (..., 4) uint32, key: (2,) or (..., 2) uint32.

    Returns (..., 4) uint32.
    """
    c = np.asarray(counter, dtype=np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0, k1 = k[..., 0], k[..., 1]
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _PHILOX_W0) & _MASK32
            k1 = (k1 + _PHILOX_W1) & _MASK32
        p0 = _PHILOX_M0 * c0          # < 2^64: exact in uint64
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


STREAM_ROTATION = 1
STREAM_SKETCH = 2
STREAM_SIGNS = 3


def philox_normals(seed: int, stream: int, count: int) -> np.ndarray:
    """count standard normals from (seed, stream).

    Block i uses counter (i mod 2^32, i div 2^32, stream, 0) and key
    (seed mod 2^32, seed div 2^32).  Each block's four words (w0..w3) give four
    normals by Box-Muller: with u(w) = (w + 1/2) / 2^32,
    rho = sqrt(-2 ln u(w0)), theta = 2 pi u(w1): rho cos theta, rho sin theta,
    and likewise from (w2, w3).
    """
    nblk = (count + 3) // 4
    i = np.arange(nblk, dtype=np.uint64)
    ctr = np.stack([i & _MASK32, i >> np.uint64(32),
                    np.full(nblk, stream, np.uint64), np.zeros(nblk, np.uint64)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    w = philox4x32_10(ctr, key).astype(np.float64)
    u = (w + 0.5) * 2.0 ** -32
    out = np.empty((nblk, 4))
    for a, b in ((0, 1), (2, 3)):
        rho = np.sqrt(-2.0 * np.log(u[:, a]))
        th = 2.0 * math.pi * u[:, b]
        out[:, a] = rho * np.cos(th)
        out[:, b] = rho * np.sin(th)
    return out.reshape(-1)[:count]


def haar_rotation(d: int, seed: int) -> np.ndarray:
    """Seeded Haar-distributed orthogonal d x d matrix (fp64).

    G has i.i.d. N(0,1) entries (row-major from the rotation stream); with
    G = QR, Pi = Q diag(sign(R_ii)) (Mezzadri's sign fix makes the law Haar).
    The codec rotates with y = Pi u.
    """
    g = philox_normals(seed, STREAM_ROTATION, d * d).reshape(d, d)
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def rademacher_signs(d: int, seed: int) -> np.ndarray:
    """d signs +1 / -1 from the sign stream: sign j is +1 when bit 0 of word j
    (block j div 4, word j mod 4) is 0 and -1 when it is 1."""
    nblk = (d + 3) // 4
    i = np.arange(nblk, dtype=np.uint64)
    ctr = np.stack([i & _MASK32, i >> np.uint64(32),
                    np.full(nblk, STREAM_SIGNS, np.uint64), np.zeros(nblk, np.uint64)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    w = philox4x32_10(ctr, key).reshape(-1)[:d]
    return np.where((w & np.uint64(1)) == 0, 1.0, -1.0)


def sylvester_hadamard(d: int) -> np.ndarray:
    """Walsh-Hadamard matrix of order d (a power of two) by Sylvester's
    doubling, H_2n = [[H_n, H_n], [H_n, -H_n]] from H_1 = [1]; entry (i, j)
    is (-1)^popcount(i & j)."""
    if d < 1 or d & (d - 1):
        raise ValueError("the Walsh-Hadamard order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_rotation(d: int, seed: int) -> np.ndarray:
    """Randomized Hadamard rotation Pi = H diag(s) / sqrt(d) (fp64): the
    reference cache's O(d log d) rotation mode (OnlyTerp/turboquant launch
    post, repository layout; the summary's "random Hadamard rotation"), with
    seeded Rademacher signs s.  Orthogonal because H H^T = d I."""
    return sylvester_hadamard(d) * rademacher_signs(d, seed)[None, :] / math.sqrt(d)


def gaussian_sketch(m: int, seed: int) -> np.ndarray:
    """Seeded m x m matrix with i.i.d. N(0, 1) entries (fp64), row-major from the sketch stream."""
    return philox_normals(seed, STREAM_SKETCH, m * m).reshape(m, m)


def stored_sketch(m: int, seed: int) -> np.ndarray:
    """The sketch S as the codec stores it: the Gaussian draws rounded to fp32
    and then to fp16 (round to nearest even each time), held in fp64.  The
    QJL estimator is exactly unbiased for Gaussian rows; the fp16 rounding
    (relative 2^-11 per entry) perturbs that by far less than the estimator's
    own spread, which the Monte-Carlo test over sketches checks."""
    g = gaussian_sketch(m, seed)
    return g.astype(np.float32).astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# Lloyd-Max codebooks.  The coordinate T of a uniformly random unit vector in
# R^d has density f_d(t) = (1 - t^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1],
# i.e. (T+1)/2 ~ Beta((d-1)/2, (d-1)/2): the "known Beta distribution" of the
# paper review's "Method", which tends to N(0, 1/d).  The cell moments are
# written in closed form (regularised incomplete beta function).
# ---------------------------------------------------------------------------
def beta_cell_moments(a, b, d: int):
    """Return (P, M1, M2) = integrals of (1, t, t^2) f_d(t) over [a, b]."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    al = (d - 1) / 2.0
    sa, sb = (a + 1) / 2, (b + 1) / 2
    p = special.betainc(al, al, sb) - special.betainc(al, al, sa)
    # t (1-t^2)^k has antiderivative -(1-t^2)^(k+1) / (2(k+1)), k = (d-3)/2.
    logb = special.betaln(0.5, al)

    def anti(t):
        with np.errstate(divide="ignore"):
            v = -np.exp(al * np.log1p(-t * t) - logb) / (2 * al)
        return np.where(np.abs(t) >= 1.0, 0.0, v)

    m1 = anti(b) - anti(a)
    # By parts: int t^2 f_d = [-t (1-t^2) f_d(t) / (d-1)] + (1/d) P_{d+2}, where
    # P_{d+2} is the cell mass under the law at dimension d+2 (Beta(al+1, al+1)).
    def edge(t):
        with np.errstate(divide="ignore"):
            v = t * np.exp(al * np.log1p(-t * t) - logb) / (d - 1)
        return np.where(np.abs(t) >= 1.0, 0.0, v)

    p2 = special.betainc(al + 1, al + 1, sb) - special.betainc(al + 1, al + 1, sa)
    m2 = edge(a) - edge(b) + p2 / d
    return p, m1, m2


def gaussian_cell_moments(a, b):
    """(P, M1, M2) of the standard normal over [a, b] (closed forms)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    phi = lambda t: np.where(np.isinf(t), 0.0, np.exp(-0.5 * np.where(np.isinf(t), 0.0, t) ** 2)
                             / math.sqrt(2 * math.pi))
    p = special.ndtr(b) - special.ndtr(a)
    m1 = phi(a) - phi(b)
    ta = np.where(np.isinf(a), 0.0, a)
    tb = np.where(np.isinf(b), 0.0, b)
    m2 = p + ta * phi(a) - tb * phi(b)
    return p, m1, m2


@dataclass
class LloydMax:
    centroids: np.ndarray      # fp64, ascending, length L
    boundaries: np.ndarray     # fp64, length L-1 (midpoints)
    mse: float                 # E[(T - Q(T))^2] per coordinate
    iterations: int


def lloyd_max(moments, lo: float, hi: float, levels: int, init: np.ndarray,
              rtol: float = 1e-16, max_iter: int = 200000, patience: int = 500) -> LloydMax:
    """Lloyd's iteration for a scalar law on [lo, hi]: boundaries at centroid
    midpoints, centroids at the conditional mean of their cell ("continuous 1-D
    k-means", paper review, "Method").  Stops when the largest centroid move is
    below rtol * max|c| (1e-16: in practice the rounding floor), or when the
    move has not reached a new minimum for
    ``patience`` steps (the rounding floor of the moments, ~1e-14).  The result
    is made exactly symmetric."""
    c = np.array(init, dtype=np.float64)
    it, best, best_it = 0, np.inf, 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[1:] + c[:-1])
        edges = np.concatenate([[lo], t, [hi]])
        p, m1, _ = moments(edges[:-1], edges[1:])
        new = m1 / p
        delta = np.max(np.abs(new - c))
        c = new
        if delta < best:
            best, best_it = delta, it
        if delta < rtol * np.max(np.abs(c)) or it - best_it > patience:
            break
    c = 0.5 * (c - c[::-1])                      # symmetric law -> symmetric codebook
    t = 0.5 * (c[1:] + c[:-1])
    if levels % 2 == 0:
        t[levels // 2 - 1] = 0.0
    edges = np.concatenate([[lo], t, [hi]])
    p, m1, m2 = moments(edges[:-1], edges[1:])
    mse = float(np.sum(m2 - 2 * c * m1 + c * c * p))
    return LloydMax(c, t, mse, it)


def beta_codebook(d: int, bits: int) -> LloydMax:
    """Lloyd-Max codebook with 2^bits levels for the rotated-coordinate law at dimension d."""
    levels = 1 << bits
    sigma = 1.0 / math.sqrt(d)
    q = special.ndtri((np.arange(levels) + 0.5) / levels) * sigma
    init = np.clip(q, -0.999, 0.999)
    return lloyd_max(lambda a, b: beta_cell_moments(a, b, d), -1.0, 1.0, levels, init)


def gaussian_codebook(bits: int) -> LloydMax:
    """Lloyd-Max codebook with 2^bits levels for N(0, 1)."""
    levels = 1 << bits
    init = special.ndtri((np.arange(levels) + 0.5) / levels)
    return lloyd_max(gaussian_cell_moments, -np.inf, np.inf, levels, init)


# ---------------------------------------------------------------------------
# SpectralQuant calibration: eigenbasis of the centred key covariance, sorted
# so that dim 0 carries the largest eigenvalue (SpectralQuant thread, tweet 4).
# ---------------------------------------------------------------------------
def eigenbasis(calib: np.ndarray):
    """Rows of the returned matrix are eigenvectors of the centred sample
    covariance (divisor n), eigenvalues descending; each row is flipped so that
    its entry of largest magnitude (first such index) is positive."""
    x = np.asarray(calib, dtype=np.float64)
    xc = x - x.mean(axis=0, keepdims=True)
    cov = xc.T @ xc / x.shape[0]
    lam, vec = np.linalg.eigh(cov)
    order = np.argsort(-lam, kind="stable")
    lam, vec = lam[order], vec[:, order]
    rows = vec.T.copy()
    for i in range(rows.shape[0]):
        j = int(np.argmax(np.abs(rows[i])))
        if rows[i, j] < 0:
            rows[i] = -rows[i]
    return lam, rows


# ---------------------------------------------------------------------------
# Codebook objects
# ---------------------------------------------------------------------------
@dataclass
class Codec:
    d: int
    mode: str                          # "mse" or "prod"
    bits: np.ndarray                   # per-dim index bits, shape [d]
    m: int                             # sketch dims (rotated dims 0..m-1); 0 for mse
    layout: str                        # "row" or "col"
    rot: np.ndarray                    # [H][d][d] fp32 values held in fp64
    sketch: Optional[np.ndarray]       # [m][m] fp32 values held in fp64
    centroids: List[List[np.ndarray]]  # [H][d] -> fp32 values held in fp64
    boundaries: List[List[np.ndarray]] # [H][d]
    uniform: bool = True
    extra: dict = field(default_factory=dict)

    @property
    def heads(self) -> int:
        return self.rot.shape[0]


def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def turboquant_codec(d: int, bits: int, mode: str, rot_seed: int, sketch_seed: int = 0,
                     layout: str = "row", rotation: str = "haar") -> Codec:
    """TurboQuant-mse (bits per coordinate) or TurboQuant-prod (bits-1 mse bits +
    1 QJL bit, sketch over all d rotated dims); paper review, "Method".
    rotation: "haar" (dense seeded Haar) or "hadamard" (randomized Hadamard)."""
    mse_bits = bits - 1 if mode == "prod" else bits
    if mse_bits < 1:
        raise ValueError("prod needs bits >= 2 here (at least one mse bit)")
    lm = beta_codebook(d, mse_bits)
    if rotation == "haar":
        rot = _f32(haar_rotation(d, rot_seed))[None]
    elif rotation == "hadamard":
        rot = _f32(hadamard_rotation(d, rot_seed))[None]
    else:
        raise ValueError(rotation)
    m = d if mode == "prod" else 0
    sk = stored_sketch(m, sketch_seed) if mode == "prod" else None
    c, t = _f32(lm.centroids), _f32(lm.boundaries)
    return Codec(d, mode, np.full(d, mse_bits), m, layout, rot, sk,
                 [[c] * d], [[t] * d], True, {"lloyd_max": lm})


def water_fill(lam, total_bits: int, min_bits: int = 1, max_bits: int = 5) -> np.ndarray:
    """Discrete reverse water-filling of index bits over dims of variance lam
    (SpectralQuant thread, tweet 6: water-filling, after Shannon and Berger,
    puts more bits on the dominant dims).  Reading: the distortion of dim i
    at b bits is lam_i D(b), D the b-bit Gaussian Lloyd-Max error; every dim
    starts at min_bits and each further bit goes to the dim whose distortion
    drops the most (ties to the lower dim) until total_bits are spent."""
    lam = np.asarray(lam, dtype=np.float64)
    d = len(lam)
    if not (d * min_bits <= total_bits <= d * max_bits):
        raise ValueError("budget outside [d min_bits, d max_bits]")
    D = {b: gaussian_codebook(b).mse for b in range(min_bits, max_bits + 1)}
    bits = np.full(d, min_bits, dtype=np.int64)
    for _ in range(total_bits - d * min_bits):
        best, gain = -1, -1.0
        for i in range(d):
            if bits[i] < max_bits:
                g = lam[i] * (D[bits[i]] - D[bits[i] + 1])
                if g > gain:
                    best, gain = i, g
        bits[best] += 1
    return bits


def spectralquant_codec(calib: np.ndarray, bitmap, m: int, sketch_seed: int,
                        layout: str = "row", waterfill_bits: int = 0) -> Codec:
    """SpectralQuant keys: per-head eigenbasis rotation, water-filled bit map
    (e.g. [5,3,2,2] on the top-4 dims, 1 bit elsewhere) and QJL on the first m
    rotated dims (SpectralQuant thread, tweets 4, 5, 6).

    Per-dim codebook: Gaussian Lloyd-Max with b_i bits scaled by sigma_i, the RMS
    of the i-th rotated coordinate of the normalised calibration vectors.

    calib: [H][n][d] calibration keys.  With bitmap None and waterfill_bits > 0
    the bit map is water_fill(lambda, waterfill_bits) with lambda_i = sigma_i^2
    averaged over the heads.
    """
    calib = np.asarray(calib, dtype=np.float64)
    heads, _, d = calib.shape
    rots, sig = [], []
    for h in range(heads):
        _, rows = eigenbasis(calib[h])
        p = _f32(rows)
        x = calib[h]
        u = x / np.linalg.norm(x, axis=1, keepdims=True)
        y = dot_rows(u, p)                        # y = P u per row
        rots.append(p)
        sig.append(np.sqrt(np.mean(y * y, axis=0)))
    if bitmap is None:
        bits = water_fill(np.mean(np.stack(sig) ** 2, axis=0), waterfill_bits)
    else:
        bits = np.asarray(bitmap, dtype=np.int64)
    books = {b: gaussian_codebook(int(b)) for b in set(bits.tolist())}
    cents, bnds = [], []
    for h in range(heads):
        sigma = sig[h]
        cents.append([_f32(books[int(bits[i])].centroids * sigma[i]) for i in range(d)])
        bnds.append([_f32(books[int(bits[i])].boundaries * sigma[i]) for i in range(d)])
    sk = stored_sketch(m, sketch_seed)
    return Codec(d, "prod", bits, m, layout, np.stack(rots), sk, cents, bnds, False,
                 {"sigma": np.stack(sig)})


# ---------------------------------------------------------------------------
# Encode
# ---------------------------------------------------------------------------
@dataclass
class Encoded:
    idx: np.ndarray                 # [n][d] int
    signs: Optional[np.ndarray]     # [n][m] bool (True = z >= 0)
    nx: np.ndarray                  # [n] fp16
    nr: Optional[np.ndarray]        # [n] fp16
    y: np.ndarray                   # [n][d] rotated unit vectors (fp64), for band checks
    z: Optional[np.ndarray]         # [n][m] sketch values (fp64)


def quantize(codec: Codec, y: np.ndarray, head: int) -> np.ndarray:
    """idx_i = number of boundaries t with t <= y_i (ties go to the upper cell)."""
    n, d = y.shape
    if codec.uniform:
        return count_le(codec.boundaries[head][0], y.reshape(-1)).reshape(n, d)
    idx = np.empty((n, d), dtype=np.int64)
    for i in range(d):
        idx[:, i] = count_le(codec.boundaries[head][i], y[:, i])
    return idx


def dequantize(codec: Codec, idx: np.ndarray, head: int) -> np.ndarray:
    n, d = idx.shape
    if codec.uniform:
        return codec.centroids[head][0][idx]
    out = np.empty((n, d))
    for i in range(d):
        out[:, i] = codec.centroids[head][i][idx[:, i]]
    return out


def encode(codec: Codec, x: np.ndarray, head: int = 0, round_norms: bool = True) -> Encoded:
    """TurboQuant encode of the rows of x (paper review, "Method").

    Norms are stored as fp16 (round to nearest even); round_norms=False keeps
    them in fp64 for statistical checks of the estimator itself."""
    x = np.asarray(x, dtype=np.float64)
    nx = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(nx > 0, nx, 1.0)
    u = np.where(nx[:, None] > 0, x / safe[:, None], 0.0)
    y = dot_rows(u, codec.rot[head])              # y = Pi u
    idx = quantize(codec, y, head)
    store = (lambda v: v.astype(np.float16)) if round_norms else (lambda v: v)
    if codec.mode == "mse":
        return Encoded(idx, None, store(nx), None, y, None)
    nr, z = residual_sketch(codec, y, idx, head)
    return Encoded(idx, z >= 0, store(nx), store(nr), y, z)


def residual_sketch(codec: Codec, y: np.ndarray, idx: np.ndarray, head: int = 0):
    """The QJL stage of TurboQuant-prod for given codes (paper review,
    "Method"): the residual r = y - c[idx] on dims 0..m-1, its norm n_r (fp64)
    and the sketch z = S r, whose signs are stored.  encode() calls it with its
    own codes; the comparison rules call it with another quantizer's codes."""
    m = codec.m
    chat = dequantize(codec, idx, head)
    r = y[:, :m] - chat[:, :m]                   # residual of the mse stage
    nr = np.sqrt(np.sum(r * r, axis=1))
    z = dot_rows(r, codec.sketch)                # S r
    return nr, z


def boundary_distance(codec: Codec, y: np.ndarray, head: int = 0) -> np.ndarray:
    """min_t |y_i - t| over the decision boundaries of dim i."""
    n, d = y.shape
    out = np.full((n, d), np.inf)
    for i in range(d):
        t = codec.boundaries[head][0 if codec.uniform else i]
        if len(t):
            out[:, i] = np.min(np.abs(y[:, i:i + 1] - t[None, :]), axis=1)
        if codec.uniform:
            out[:] = np.min(np.abs(y[:, :, None] - t[None, None, :]), axis=2)
            break
    return out


# ---------------------------------------------------------------------------
# Scoring (two independent paths) and decode attention
# ---------------------------------------------------------------------------
QJL_CONST = math.sqrt(math.pi / 2)


def prepare_query(codec: Codec, q: np.ndarray, head: int = 0):
    """q' = Pi q and (prod) q_s = S q'[0:m]."""
    q = np.asarray(q, dtype=np.float64)
    qr = dot_rows(q, codec.rot[head])
    qs = dot_rows(qr[:, :codec.m], codec.sketch) if codec.mode == "prod" else None
    return qr, qs


def score(codec: Codec, q: np.ndarray, enc: Encoded, head: int = 0) -> np.ndarray:
    """s = n_x (sum_i q'_i c[idx_i] + n_r sqrt(pi/2)/m sum_j q_s,j (2 bit_j - 1)).

    [nq][n] scores with the stored (fp16) norms."""
    qr, qs = prepare_query(codec, q, head)
    chat = dequantize(codec, enc.idx, head)
    nx = enc.nx.astype(np.float64)
    s = dot_rows(qr, chat)
    if codec.mode == "prod":
        pm = np.where(enc.signs, 1.0, -1.0)
        s = s + dot_rows(qs, pm) * (enc.nr.astype(np.float64) * QJL_CONST / codec.m)[None, :]
    return s * nx[None, :]


def reconstruct(codec: Codec, enc: Encoded, head: int = 0) -> np.ndarray:
    """x_hat = n_x Pi^T (c[idx] + n_r sqrt(pi/2)/m [S^T sign ; 0])."""
    chat = dequantize(codec, enc.idx, head)
    if codec.mode == "prod":
        pm = np.where(enc.signs, 1.0, -1.0)
        corr = dot_rows(pm, codec.sketch.T) * (enc.nr.astype(np.float64) * QJL_CONST / codec.m)[:, None]
        chat = chat.copy()
        chat[:, :codec.m] += corr
    return dot_rows(chat, codec.rot[head].T) * enc.nx.astype(np.float64)[:, None]


def score_via_reconstruction(codec: Codec, q: np.ndarray, enc: Encoded, head: int = 0):
    """Second scoring path: <q, x_hat>."""
    return dot_rows(np.asarray(q, dtype=np.float64), reconstruct(codec, enc, head))


def decode_attention(kcodec: Codec, vcodec: Codec, q: np.ndarray, kenc: List[Encoded],
                     venc: List[Encoded], scale: float, kv_heads_rot: bool = True) -> np.ndarray:
    """One decode step of grouped-query attention over a compressed cache.

    q: [Hq][d]; kenc/venc: one Encoded per KV head.  Query head h reads KV head
    h // (Hq / Hkv).  logits = scale * score; softmax over tokens; the output is
    sum_t p_t v_hat_t with v_hat the mse reconstruction."""
    hq = q.shape[0]
    hkv = len(kenc)
    group = hq // hkv
    out = np.zeros((hq, q.shape[1]))
    for h in range(hq):
        g = h // group
        kh = g if kcodec.heads > 1 else 0
        vh = g if vcodec.heads > 1 else 0
        s = score(kcodec, q[h:h + 1], kenc[g], kh)[0] * scale
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = dot_rows(p, reconstruct(vcodec, venc[g], vh).T)[0]
    return out


def topk(scores: np.ndarray, k: int):
    """Per row the k largest scores, descending; equal scores go to the smaller id."""
    nq, n = scores.shape
    ids = np.empty((nq, k), dtype=np.int64)
    for i in range(nq):
        order = np.lexsort((np.arange(n), -scores[i]))
        ids[i] = order[:k]
    return np.take_along_axis(scores, ids, axis=1), ids


# ---------------------------------------------------------------------------
# Record layout (the library's specification; the pages give none).
#
# Records are grouped in tiles of 64 vectors.  Fields of a tile, in order:
#   codes, signs (prod only), n_x (fp16 x 64), n_r (fp16 x 64, prod only).
# Row layout: a vector's code bits form one bit string, plane by plane (plane p
#   holds bit p of the index of every dim with more than p bits, dims
#   ascending); bit k is bit (k mod 8) of byte k div 8.  Its C = ceil(B/8) bytes
#   are cut into 16-byte chunks (the last may be shorter); chunk j of the tile
#   is stored as [64 vectors][width_j] bytes.  Sign bits (bit j = [z_j >= 0])
#   are packed and chunked the same way.
# Col layout (uniform codecs, b index bits): for every dim i, ascending, a field
#   of 8*b bytes holding the b-bit indices of the tile's 64 vectors, vector v at
#   bits [b*v, b*v + b) (bit k of the field is bit k mod 8 of byte k div 8);
#   then one 64-bit word per sketch dim j (bit v = sign bit of vector v).
# Slots of a partly filled last tile are zero.
# ---------------------------------------------------------------------------
TILE = 64


def plane_dims(bits: np.ndarray):
    return [np.nonzero(bits > p)[0] for p in range(int(bits.max()))]


def _chunks(nbytes: int):
    out, off = [], 0
    while off < nbytes:
        w = min(16, nbytes - off)
        out.append((off, w))
        off += w
    return out


def tile_fields(codec: Codec):
    """(field name, byte offset in tile, bytes) for every field of a tile."""
    fields, off = [], 0
    total_bits = int(codec.bits.sum())
    if codec.layout == "row":
        for j, (o, w) in enumerate(_chunks((total_bits + 7) // 8)):
            fields.append((f"code{j}", off, TILE * w))
            off += TILE * w
        if codec.mode == "prod":
            for j, (o, w) in enumerate(_chunks((codec.m + 7) // 8)):
                fields.append((f"sign{j}", off, TILE * w))
                off += TILE * w
    else:
        fields.append(("codes", off, 8 * total_bits))
        off += 8 * total_bits
        if codec.mode == "prod":
            fields.append(("signs", off, 8 * codec.m))
            off += 8 * codec.m
    fields.append(("nx", off, 2 * TILE))
    off += 2 * TILE
    if codec.mode == "prod":
        fields.append(("nr", off, 2 * TILE))
        off += 2 * TILE
    return fields


def tile_bytes(codec: Codec) -> int:
    f = tile_fields(codec)
    return f[-1][1] + f[-1][2]


def _row_bitstrings(codec: Codec, idx: np.ndarray) -> np.ndarray:
    planes = []
    for p, dims in enumerate(plane_dims(codec.bits)):
        planes.append(((idx[:, dims] >> p) & 1).astype(np.uint8))
    return np.concatenate(planes, axis=1)


def pack(codec: Codec, enc: Encoded) -> np.ndarray:
    """Bytes of ceil(n/64) tiles holding the records of enc."""
    n = enc.idx.shape[0]
    ntile = (n + TILE - 1) // TILE
    tb = tile_bytes(codec)
    buf = np.zeros(ntile * tb, dtype=np.uint8)
    fields = dict((f[0], (f[1], f[2])) for f in tile_fields(codec))
    pad = ntile * TILE - n
    idx = np.concatenate([enc.idx, np.zeros((pad, codec.d), np.int64)])
    sg = None
    if codec.mode == "prod":
        sg = np.concatenate([enc.signs, np.zeros((pad, codec.m), bool)]).astype(np.uint8)
    nx = np.concatenate([enc.nx, np.zeros(pad, np.float16)])
    nr = np.concatenate([enc.nr, np.zeros(pad, np.float16)]) if codec.mode == "prod" else None
    for t in range(ntile):
        base = t * tb
        rows = slice(t * TILE, (t + 1) * TILE)
        if codec.layout == "row":
            cbytes = np.packbits(_row_bitstrings(codec, idx[rows]), axis=1, bitorder="little")
            for j, (o, w) in enumerate(_chunks(cbytes.shape[1])):
                fo, _ = fields[f"code{j}"]
                buf[base + fo: base + fo + TILE * w] = cbytes[:, o:o + w].reshape(-1)
            if sg is not None:
                sbytes = np.packbits(sg[rows], axis=1, bitorder="little")
                for j, (o, w) in enumerate(_chunks(sbytes.shape[1])):
                    fo, _ = fields[f"sign{j}"]
                    buf[base + fo: base + fo + TILE * w] = sbytes[:, o:o + w].reshape(-1)
        else:
            b = int(codec.bits[0])
            fields_i = []
            for i in range(codec.d):
                # bit (b*v + k) of the field = bit k of the index of vector v
                bits = ((idx[rows, i][:, None] >> np.arange(b)[None, :]) & 1).astype(np.uint8)
                fields_i.append(np.packbits(bits.reshape(-1), bitorder="little"))
            fo, fl = fields["codes"]
            buf[base + fo: base + fo + fl] = np.concatenate(fields_i)
            if sg is not None:
                fo, fl = fields["signs"]
                buf[base + fo: base + fo + fl] = np.concatenate(
                    [np.packbits(sg[rows, j], bitorder="little") for j in range(codec.m)])
        fo, _ = fields["nx"]
        buf[base + fo: base + fo + 2 * TILE] = nx[rows].view(np.uint8)
        if nr is not None:
            fo, _ = fields["nr"]
            buf[base + fo: base + fo + 2 * TILE] = nr[rows].view(np.uint8)
    return buf


def unpack(codec: Codec, buf: np.ndarray, n: int) -> Encoded:
    """Inverse of pack (y and z are not stored and come back as None)."""
    buf = np.asarray(buf, dtype=np.uint8)
    ntile = (n + TILE - 1) // TILE
    tb = tile_bytes(codec)
    fields = dict((f[0], (f[1], f[2])) for f in tile_fields(codec))
    d = codec.d
    tiles = buf[:ntile * tb].reshape(ntile, tb)

    def field_rows(name, w):
        # a [64 vectors][w bytes] field of every tile, as [ntile * 64][w]
        fo, _ = fields[name]
        return tiles[:, fo:fo + TILE * w].reshape(ntile * TILE, w)

    idx = np.zeros((ntile * TILE, d), dtype=np.int64)
    sg = None
    if codec.layout == "row":
        total_bits = int(codec.bits.sum())
        nbytes = (total_bits + 7) // 8
        cb = np.concatenate([field_rows(f"code{j}", w) for j, (_, w) in enumerate(_chunks(nbytes))], axis=1)
        bitsarr = np.unpackbits(cb, axis=1, bitorder="little")[:, :total_bits]
        small = np.zeros((ntile * TILE, d), dtype=np.uint8)
        k = 0
        for p, dims in enumerate(plane_dims(codec.bits)):
            # a plane over a run of consecutive dims (every uniform codec) is a slice
            cols = slice(dims[0], dims[-1] + 1) if dims[-1] - dims[0] + 1 == len(dims) else dims
            small[:, cols] |= bitsarr[:, k:k + len(dims)] << np.uint8(p)
            k += len(dims)
        idx[:] = small
        if codec.mode == "prod":
            nb = (codec.m + 7) // 8
            sb = np.concatenate([field_rows(f"sign{j}", w) for j, (_, w) in enumerate(_chunks(nb))], axis=1)
            sg = np.unpackbits(sb, axis=1, bitorder="little")[:, :codec.m].astype(bool)
    else:
        b = int(codec.bits[0])
        if codec.mode == "prod":
            sg = np.zeros((ntile * TILE, codec.m), dtype=bool)
        for t in range(ntile):
            rows = slice(t * TILE, (t + 1) * TILE)
            fo, fl = fields["codes"]
            per_dim = tiles[t, fo:fo + fl].reshape(codec.d, 8 * b)
            for i in range(codec.d):
                bits = np.unpackbits(per_dim[i], bitorder="little").reshape(TILE, b).astype(np.int64)
                idx[rows, i] = (bits << np.arange(b)[None, :]).sum(axis=1)
            if sg is not None:
                fo, fl = fields["signs"]
                words = tiles[t, fo:fo + fl].reshape(-1, 8)
                for j in range(codec.m):
                    sg[rows, j] = np.unpackbits(words[j], bitorder="little").astype(bool)
    nx = np.ascontiguousarray(field_rows("nx", 2)).view(np.float16).reshape(-1)
    nr = np.ascontiguousarray(field_rows("nr", 2)).view(np.float16).reshape(-1) if codec.mode == "prod" else None
    return Encoded(idx[:n], None if sg is None else sg[:n], nx[:n],
                   None if nr is None else nr[:n], None, None)


# ---------------------------------------------------------------------------
# Outlier-channel split (TurboQuant paper review, "Method": for the KV-cache
# experiments the channels are divided into an outlier group and a regular
# group, each quantized by its own, independent TurboQuant instance; the
# 2.5-bit setting gives 32 outlier channels 3 bits and the other 96 channels
# 2 bits).
#
# Readings (the pages name the split and one bit budget, nothing more):
# * the outlier channels are given by the caller, per KV head (the launch kit
#   speaks of outlier channels found online and of per-model channel lists);
# * the regular instance takes the remaining channels in ascending order and
#   the seeds (rot_seed, sketch_seed); the outlier instance takes the listed
#   channels in list order and the seeds (rot_seed + 1, sketch_seed + 1);
# * both instances use the same mode; each stores its own norms.
#
# Library record layout of a split codec (d a multiple of 32): the two
# instances' rotated coordinates are interleaved.  Stored coordinate i, with
# blk = i // 32 and r = i % 32 and p = o / (d / 32) outlier coordinates per
# 32-block, is outlier coordinate blk * p + r when r < p, else regular
# coordinate blk * (32 - p) + r - p.  Codes and sign bits follow the row
# layout over the stored coordinates (per-dim bits: the outlier instance's on
# outlier coordinates); the tile's fields are codes, signs (prod), n_x and
# n_r (prod) of the regular instance, then n_x and n_r (prod) of the outlier
# instance, fp16 x 64 each.
# ---------------------------------------------------------------------------
@dataclass
class SplitCodec:
    d: int
    mode: str
    outlier: np.ndarray      # [H][o] outlier channels per head, in instance order
    regular: np.ndarray      # [H][d - o] the other channels, ascending
    inst_o: Codec            # TurboQuant instance of dimension o
    inst_r: Codec            # TurboQuant instance of dimension d - o
    layout: str = "row"      # "col": mse values in 8-token code words (split_col_layout)

    @property
    def o(self) -> int:
        return self.outlier.shape[1]

    @property
    def heads(self) -> int:
        return self.outlier.shape[0]


@dataclass
class SplitEncoded:
    o: Encoded               # outlier instance
    r: Encoded               # regular instance


def outlier_split_codec(d: int, outlier_channels, bits_outlier: int, bits_regular: int, mode: str,
                        rot_seed: int, sketch_seed: int = 0, layout: str = "row") -> SplitCodec:
    """Two independent TurboQuant instances over a channel split (paper
    review, "Method", KV-cache setting).  outlier_channels: [o] or [H][o]."""
    ch = np.atleast_2d(np.asarray(outlier_channels, dtype=np.int64))
    o = ch.shape[1]
    if not 0 < o < d:
        raise ValueError("need 0 < o < d outlier channels")
    regular = []
    for h in range(ch.shape[0]):
        s = set(ch[h].tolist())
        if len(s) != o or min(s) < 0 or max(s) >= d:
            raise ValueError("outlier channels must be distinct and in [0, d)")
        regular.append([c for c in range(d) if c not in s])
    if layout not in ("row", "col") or (layout == "col" and (mode != "mse" or d != 128)):
        raise ValueError("the col layout of a split codec holds d = 128 mse values")
    inst_o = turboquant_codec(o, bits_outlier, mode, rot_seed + 1, sketch_seed + 1)
    inst_r = turboquant_codec(d - o, bits_regular, mode, rot_seed, sketch_seed)
    return SplitCodec(d, mode, ch, np.asarray(regular, dtype=np.int64), inst_o, inst_r, layout)


# Col layout of split values (d = 128, mse; the library's layout, written
# out here from its specification): per tile, for each 8-token group g
# (tokens 8g .. 8g + 7) the 16 lane blocks n = 0..15 in order, block n holding
# stored coordinates 16 vb + n for vb = 0..7 in that order, coordinate i as a
# little-endian word of b_i bytes whose bits b_i k .. b_i k + b_i - 1 are the
# index of token 8g + k (b_i: its index bits).  Then n_x of the regular and
# of the outlier instance, fp16 x 64 each.
def split_col_layout(bits):
    """(offset of coordinate i's word within a token group [d], group bytes)."""
    bits = np.asarray(bits, dtype=np.int64)
    off = np.zeros(len(bits), dtype=np.int64)
    pos = 0
    for n in range(16):
        for vb in range(8):
            i = 16 * vb + n
            off[i] = pos
            pos += int(bits[i])
    return off, pos


def split_encode(sc: SplitCodec, x: np.ndarray, head: int = 0, round_norms: bool = True) -> SplitEncoded:
    """Each channel group encoded by its own instance."""
    x = np.asarray(x, dtype=np.float64)
    return SplitEncoded(encode(sc.inst_o, x[:, sc.outlier[head]], 0, round_norms),
                        encode(sc.inst_r, x[:, sc.regular[head]], 0, round_norms))


def split_score(sc: SplitCodec, q: np.ndarray, enc: SplitEncoded, head: int = 0) -> np.ndarray:
    """<q, x> estimated as the sum of the two instances' estimates over their channels."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    return (score(sc.inst_o, q[:, sc.outlier[head]], enc.o)
            + score(sc.inst_r, q[:, sc.regular[head]], enc.r))


def split_reconstruct(sc: SplitCodec, enc: SplitEncoded, head: int = 0) -> np.ndarray:
    """x_hat with each channel group reconstructed by its instance."""
    n = enc.o.idx.shape[0]
    out = np.zeros((n, sc.d))
    out[:, sc.outlier[head]] = reconstruct(sc.inst_o, enc.o)
    out[:, sc.regular[head]] = reconstruct(sc.inst_r, enc.r)
    return out


def split_decode_attention(kcodec, vcodec, q: np.ndarray, kenc: list, venc: list,
                           scale: float) -> np.ndarray:
    """decode_attention with keys and/or values of a split codec (either may
    also be a plain Codec).  Query head h reads KV head h // (Hq / Hkv); a
    codec with one head serves every KV head."""
    def sc_(codec, qq, enc, g):
        if isinstance(codec, SplitCodec):
            return split_score(codec, qq, enc, g if codec.heads > 1 else 0)
        return score(codec, qq, enc, g if codec.heads > 1 else 0)

    def rec_(codec, enc, g):
        if isinstance(codec, SplitCodec):
            return split_reconstruct(codec, enc, g if codec.heads > 1 else 0)
        return reconstruct(codec, enc, g if codec.heads > 1 else 0)

    hq = q.shape[0]
    group = hq // len(kenc)
    out = np.zeros((hq, q.shape[1]))
    for h in range(hq):
        g = h // group
        s = sc_(kcodec, q[h:h + 1], kenc[g], g)[0] * scale
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = dot_rows(p, rec_(vcodec, venc[g], g).T)[0]
    return out


def split_stored_order(d: int, o: int):
    """(group [d], coord [d]): stored coordinate i holds coordinate coord[i] of
    the outlier instance (group 1) or of the regular instance (group 0)."""
    if d % 32 or (o * 32) % d:
        raise ValueError("the interleaved layout needs d % 32 == 0 and o a multiple of d / 32")
    p = o * 32 // d
    group = np.zeros(d, dtype=np.int64)
    coord = np.zeros(d, dtype=np.int64)
    for i in range(d):
        blk, r = divmod(i, 32)
        if r < p:
            group[i], coord[i] = 1, blk * p + r
        else:
            group[i], coord[i] = 0, blk * (32 - p) + r - p
    return group, coord


def split_stored_codec(sc: SplitCodec) -> Codec:
    """The split codec seen as one d-dim codec in stored order: rotation rows
    of head h = the instances' rotation rows placed on their channels, the
    block-diagonal sketch, per-dim bits and codebooks.  (The library holds a
    split codec in this form; the oracle itself encodes and scores with the
    two instances.)"""
    d = sc.d
    group, coord = split_stored_order(d, sc.o)
    rot = np.zeros((sc.heads, d, d))
    for h in range(sc.heads):
        for i in range(d):
            if group[i]:
                rot[h, i, sc.outlier[h]] = sc.inst_o.rot[0][coord[i]]
            else:
                rot[h, i, sc.regular[h]] = sc.inst_r.rot[0][coord[i]]
    inst = [sc.inst_r, sc.inst_o]
    bits = np.array([int(inst[group[i]].bits[coord[i]]) for i in range(d)], dtype=np.int64)
    sk = None
    if sc.mode == "prod":
        sk = np.zeros((d, d))
        for i in range(d):
            for j in range(d):
                if group[i] == group[j]:
                    sk[i, j] = inst[group[i]].sketch[coord[i], coord[j]]
    cents = [[inst[group[i]].centroids[0][0] for i in range(d)]] * sc.heads
    bnds = [[inst[group[i]].boundaries[0][0] for i in range(d)]] * sc.heads
    return Codec(d, sc.mode, bits, d if sc.mode == "prod" else 0, "row", rot, sk, cents, bnds, False,
                 {"group": group, "coord": coord})


def _split_stored_encoded(sc: SplitCodec, enc: SplitEncoded) -> Encoded:
    group, coord = split_stored_order(sc.d, sc.o)
    parts = [enc.r, enc.o]
    n = enc.o.idx.shape[0]
    idx = np.zeros((n, sc.d), dtype=np.int64)
    signs = np.zeros((n, sc.d), dtype=bool) if sc.mode == "prod" else None
    for i in range(sc.d):
        idx[:, i] = parts[group[i]].idx[:, coord[i]]
        if signs is not None:
            signs[:, i] = parts[group[i]].signs[:, coord[i]]
    return Encoded(idx, signs, enc.r.nx, enc.r.nr, None, None)


def split_tile_fields(sc: SplitCodec):
    """tile_fields of the stored-order codec (col: the code words, then n_x),
    then the outlier instance's norms."""
    if sc.layout == "col":
        _, gbytes = split_col_layout(split_stored_codec(sc).bits)
        return [("codes", 0, 8 * gbytes), ("nx", 8 * gbytes, 2 * TILE), ("nx_o", 8 * gbytes + 2 * TILE, 2 * TILE)]
    fields = tile_fields(split_stored_codec(sc))
    off = fields[-1][1] + fields[-1][2]
    fields.append(("nx_o", off, 2 * TILE))
    if sc.mode == "prod":
        fields.append(("nr_o", off + 2 * TILE, 2 * TILE))
    return fields


def split_tile_bytes(sc: SplitCodec) -> int:
    f = split_tile_fields(sc)
    return f[-1][1] + f[-1][2]


def _split_col_pack(sc: SplitCodec, enc: SplitEncoded) -> np.ndarray:
    stored = split_stored_codec(sc)
    st = _split_stored_encoded(sc, enc)
    off, gbytes = split_col_layout(stored.bits)
    n = st.idx.shape[0]
    ntile = (n + TILE - 1) // TILE
    tb = split_tile_bytes(sc)
    fields = dict((f[0], f[1]) for f in split_tile_fields(sc))
    pad = ntile * TILE - n
    idx = np.concatenate([st.idx, np.zeros((pad, sc.d), np.int64)])
    nx = np.concatenate([enc.r.nx, np.zeros(pad, np.float16)])
    nxo = np.concatenate([enc.o.nx, np.zeros(pad, np.float16)])
    buf = np.zeros(ntile * tb, dtype=np.uint8)
    for t in range(ntile):
        base = t * tb
        for g in range(8):
            for i in range(sc.d):
                b = int(stored.bits[i])
                word = 0
                for k in range(8):
                    word |= int(idx[t * TILE + 8 * g + k, i]) << (b * k)
                for j in range(b):
                    buf[base + g * gbytes + off[i] + j] = (word >> (8 * j)) & 0xFF
        rows = slice(t * TILE, (t + 1) * TILE)
        buf[base + fields["nx"]: base + fields["nx"] + 2 * TILE] = nx[rows].view(np.uint8)
        buf[base + fields["nx_o"]: base + fields["nx_o"] + 2 * TILE] = nxo[rows].view(np.uint8)
    return buf


def _split_col_unpack(sc: SplitCodec, buf: np.ndarray, n: int) -> SplitEncoded:
    stored = split_stored_codec(sc)
    off, gbytes = split_col_layout(stored.bits)
    ntile = (n + TILE - 1) // TILE
    tb = split_tile_bytes(sc)
    fields = dict((f[0], f[1]) for f in split_tile_fields(sc))
    idx = np.zeros((ntile * TILE, sc.d), dtype=np.int64)
    nx = np.zeros(ntile * TILE, np.float16)
    nxo = np.zeros(ntile * TILE, np.float16)
    for t in range(ntile):
        base = t * tb
        for g in range(8):
            for i in range(sc.d):
                b = int(stored.bits[i])
                word = 0
                for j in range(b):
                    word |= int(buf[base + g * gbytes + off[i] + j]) << (8 * j)
                for k in range(8):
                    idx[t * TILE + 8 * g + k, i] = (word >> (b * k)) & ((1 << b) - 1)
        nx[t * TILE:(t + 1) * TILE] = buf[base + fields["nx"]: base + fields["nx"] + 2 * TILE].view(np.float16)
        nxo[t * TILE:(t + 1) * TILE] = buf[base + fields["nx_o"]: base + fields["nx_o"] + 2 * TILE].view(np.float16)
    group, coord = split_stored_order(sc.d, sc.o)
    out = []
    for gsel in (1, 0):
        cols = np.nonzero(group == gsel)[0]
        order = cols[np.argsort(coord[cols])]
        out.append(idx[:n, order])
    return SplitEncoded(Encoded(out[0], None, nxo[:n], None, None, None),
                        Encoded(out[1], None, nx[:n], None, None, None))


def split_pack(sc: SplitCodec, enc: SplitEncoded) -> np.ndarray:
    """Bytes of the record tiles of a split codec (layout above)."""
    if sc.layout == "col":
        return _split_col_pack(sc, enc)
    stored = split_stored_codec(sc)
    inner = pack(stored, _split_stored_encoded(sc, enc))
    tb_in, tb = tile_bytes(stored), split_tile_bytes(sc)
    n = enc.o.idx.shape[0]
    ntile = (n + TILE - 1) // TILE
    fields = dict((f[0], f[1]) for f in split_tile_fields(sc))
    pad = ntile * TILE - n
    nxo = np.concatenate([enc.o.nx, np.zeros(pad, np.float16)])
    nro = np.concatenate([enc.o.nr, np.zeros(pad, np.float16)]) if sc.mode == "prod" else None
    buf = np.zeros(ntile * tb, dtype=np.uint8)
    for t in range(ntile):
        rows = slice(t * TILE, (t + 1) * TILE)
        buf[t * tb: t * tb + tb_in] = inner[t * tb_in: (t + 1) * tb_in]
        buf[t * tb + fields["nx_o"]: t * tb + fields["nx_o"] + 2 * TILE] = nxo[rows].view(np.uint8)
        if nro is not None:
            buf[t * tb + fields["nr_o"]: t * tb + fields["nr_o"] + 2 * TILE] = nro[rows].view(np.uint8)
    return buf


def split_unpack(sc: SplitCodec, buf: np.ndarray, n: int) -> SplitEncoded:
    """Inverse of split_pack (y and z come back as None)."""
    buf = np.asarray(buf, dtype=np.uint8)
    if sc.layout == "col":
        return _split_col_unpack(sc, buf, n)
    stored = split_stored_codec(sc)
    tb_in, tb = tile_bytes(stored), split_tile_bytes(sc)
    ntile = (n + TILE - 1) // TILE
    fields = dict((f[0], f[1]) for f in split_tile_fields(sc))
    inner = np.concatenate([buf[t * tb: t * tb + tb_in] for t in range(ntile)])
    st = unpack(stored, inner, n)
    nxo = np.concatenate([buf[t * tb + fields["nx_o"]: t * tb + fields["nx_o"] + 2 * TILE]
                          for t in range(ntile)]).view(np.float16)[:n]
    nro = None
    if sc.mode == "prod":
        nro = np.concatenate([buf[t * tb + fields["nr_o"]: t * tb + fields["nr_o"] + 2 * TILE]
                              for t in range(ntile)]).view(np.float16)[:n]
    group, coord = split_stored_order(sc.d, sc.o)
    out = []
    for gsel, inst in ((1, sc.inst_o), (0, sc.inst_r)):
        cols = np.nonzero(group == gsel)[0]
        order = cols[np.argsort(coord[cols])]
        idx = st.idx[:, order]
        sg = st.signs[:, order] if st.signs is not None else None
        out.append((idx, sg))
    enc_o = Encoded(out[0][0], out[0][1], nxo, nro, None, None)
    enc_r = Encoded(out[1][0], out[1][1], st.nx, st.nr, None, None)
    return SplitEncoded(enc_o, enc_r)
