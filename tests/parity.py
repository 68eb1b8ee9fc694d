"""Comparison rules between the HIP path and the oracle.

* codes: bit-exact except coordinates whose rotated value lies within 1e-5 of
  a decision boundary (measured on the oracle's y), which are counted;
* signs and n_r of a vector depend on all its codes: for a vector with such a
  flip, the oracle recomputes its residual, n_r and sketch z from the GPU's
  codes (and its own rotated values) before comparing; signs may then differ
  only where |z| < 1e-5;
* norms are fp16: equal up to one unit in the last place (both sides round a
  value that agrees to ~1e-7 relative, so only round-half cases can differ);
* scores within 1e-3 * ||q|| * n_x, attention outputs within 1e-3 * max n_v
  (the 1e-3 unit-scaled tolerance).
"""
import numpy as np

from oracle import tq_oracle as o

BAND = 1e-5


def fp16_ulps(a, b):
    a = np.asarray(a, np.float16).view(np.int16).astype(np.int32)
    b = np.asarray(b, np.float16).view(np.int16).astype(np.int32)
    return np.abs(a - b)


def check_encoded(codec, ref, got, band=BAND, head=0):
    """Assert the comparison rules; return counts for reporting.  `head`
    selects the codebook head whose boundaries define the band."""
    near = o.boundary_distance(codec, ref.y, head) < band
    flips = got.idx != ref.idx
    bad = flips & ~near
    assert not bad.any(), f"{int(bad.sum())} code(s) differ away from any boundary, first at " \
                          f"{np.argwhere(bad)[:3].tolist()}"
    vflip = flips.any(axis=1)
    assert np.all(fp16_ulps(got.nx, ref.nx) <= 1), "n_x differs by more than 1 fp16 ulp"
    stats = {"vectors": int(ref.idx.shape[0]), "band_code_flips": int(flips.sum()),
             "vectors_with_flips": int(vflip.sum())}
    if ref.signs is not None:
        z, nr = ref.z, ref.nr
        if vflip.any():
            # the cascade: r, n_r and z of these vectors follow the GPU's codes
            z = z.copy()
            nr = nr.copy()
            rows = np.nonzero(vflip)[0]
            nr_c, z_c = o.residual_sketch(codec, ref.y[rows], got.idx[rows], head)
            z[rows] = z_c
            nr[rows] = nr_c.astype(np.float16)
        smis = got.signs != (z >= 0)
        smis_far = smis & (np.abs(z) >= band)
        assert not smis_far.any(), f"{int(smis_far.sum())} sign bit(s) differ with |z| >= {band}: " \
                                   f"|z| = {np.abs(z[smis_far])[:5].tolist()}"
        assert np.all(fp16_ulps(got.nr, nr) <= 1), "n_r differs by more than 1 fp16 ulp"
        stats["band_sign_flips"] = int(smis.sum())
    return stats


def check_scores(got, ref_scores, q, nx):
    tol = 1e-3 * np.linalg.norm(np.asarray(q, np.float64), axis=1)[:, None] * \
        np.asarray(nx, np.float64)[None, :]
    err = np.abs(np.asarray(got, np.float64) - ref_scores)
    assert np.all(err <= tol + 1e-30), f"max scaled error {np.max(err / (tol + 1e-30)):.3g}"
    return float(np.max(err / (tol + 1e-30)))
