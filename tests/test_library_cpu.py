"""CPU checks of the C-ABI library: it loads, exports every declared entry
point, its host-side builder (Pi, S, Lloyd-Max tables, eigenbasis) agrees with
the oracle's independent implementation, and argument errors are reported
before anything is launched.  No kernel runs here."""
import ctypes
import os
import re
import sys

import numpy as np
import pytest
import torch

import kv_cache_compression_encode_amd as tq
from kv_cache_compression_encode_amd import _lib as L
from oracle import tq_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "tq.h")) as f:
        hdr = f.read()
    declared = set(re.findall(r"^\s*(?:tq_status|int64_t|size_t|const char\*)\s+(tq_\w+)\(", hdr, re.M))
    assert declared == set(L.EXPORTED)
    lib = L.lib()
    for name in declared:
        assert hasattr(lib, name)


def _ulp_mismatch(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    diff = np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))
    return int((diff > 0).sum()), int(diff.max())


@pytest.mark.parametrize("d", [8, 128])
def test_rotation_and_sketch_match_oracle(d):
    cb = tq.Codebook(d, tq.TQ_PROD, 3, seed_rotation=303, seed_sketch=304, device=-1)
    rot, sk, cen, thr, lv = cb.export()
    ref_rot = o.haar_rotation(d, 303).astype(np.float32)
    n, mx = _ulp_mismatch(rot, ref_rot)
    assert mx <= 1 and n <= 2
    ref_sk = o.stored_sketch(d, 304).astype(np.float32)
    n, mx = _ulp_mismatch(sk, ref_sk)
    assert mx <= 1 and n <= 2


@pytest.mark.parametrize("d,seed", [(8, 5), (128, 203), (1024, 9)])
def test_hadamard_rotation_matches_oracle(d, seed):
    cb = tq.Codebook(d, tq.TQ_PROD, 3, rotation=tq.TQ_ROT_HADAMARD, seed_rotation=seed, seed_sketch=4,
                     device=-1)
    rot = cb.export()[0]
    assert np.array_equal(rot, o.hadamard_rotation(d, seed).astype(np.float32))
    with pytest.raises(tq.TQError):
        tq.Codebook(96, tq.TQ_MSE, 2, rotation=tq.TQ_ROT_HADAMARD, device=-1)


def test_water_fill_matches_oracle():
    rng = np.random.default_rng(9)
    for d, total in ((4, 12), (128, 136), (128, 200), (64, 300)):
        lam = rng.gamma(0.4, size=d)
        assert np.array_equal(tq.water_fill(lam, total), o.water_fill(lam, total))
    with pytest.raises(tq.TQError):
        tq.water_fill([1.0, 2.0], 1)
    with pytest.raises(tq.TQError):
        tq.water_fill([1.0, -2.0], 4)


def test_water_filled_codebook_matches_oracle():
    import synth, torch
    law = synth.KVLaw(2, 128, 405)
    calib = torch.stack([law.sample(h, 512, torch.Generator().manual_seed(405 + h), "cpu") for h in range(2)])
    cb = tq.Codebook(128, tq.TQ_PROD, 0, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE, num_heads=2,
                     seed_sketch=404, calib=calib, waterfill_bits=136, device=-1)
    ref = o.spectralquant_codec(calib.float().numpy().astype(np.float64), None, 4, sketch_seed=404,
                                waterfill_bits=136)
    for h in range(2):
        _, _, cen, thr, lv = cb.export(h)
        assert np.array_equal(lv, 1 << ref.bits)
        for i in range(128):
            L = lv[i]
            assert np.allclose(cen[i, :L], ref.centroids[h][i], rtol=1e-6, atol=1e-9)


def test_rotation_matches_oracle_d1536():
    cb = tq.Codebook(1536, tq.TQ_MSE, 2, seed_rotation=503, device=-1)
    rot = cb.export()[0]
    ref = o.haar_rotation(1536, 503).astype(np.float32)
    n, mx = _ulp_mismatch(rot, ref)
    assert mx <= 1 and n <= 50


@pytest.mark.parametrize("d,bits,mode", [(8, 2, tq.TQ_MSE), (128, 3, tq.TQ_PROD), (128, 4, tq.TQ_MSE),
                                         (128, 5, tq.TQ_MSE), (1536, 2, tq.TQ_PROD), (1536, 4, tq.TQ_PROD)])
def test_codebook_matches_oracle(d, bits, mode):
    cb = tq.Codebook(d, mode, bits, seed_rotation=1, seed_sketch=2, device=-1)
    _, _, cen, thr, lv = cb.export()
    ub = bits - 1 if mode == tq.TQ_PROD else bits
    ref = o.beta_codebook(d, ub)
    L_ = 1 << ub
    assert np.all(lv == L_)
    # two quadratures of the same fixed point; at d = 1536 the incomplete beta
    # function near parameter 767 limits the oracle to ~1e-12
    tol = 1e-13 if d <= 128 else 1e-11
    assert np.max(np.abs(cen[0, :L_] - ref.centroids)) < tol
    assert np.max(np.abs(thr[0, :L_ - 1] - ref.boundaries)) < tol
    assert np.all(cen[:, :L_] == cen[0, :L_])


def test_spectralquant_calibration_matches_oracle():
    import synth
    law = synth.KVLaw(2, 128, 405)
    g = torch.Generator().manual_seed(7)
    calib = torch.stack([law.sample(h, 2048, g, "cpu") for h in range(2)])  # bf16 [2][2048][128]
    bitmap = [5, 3, 2, 2] + [1] * 124
    cb = tq.Codebook(128, tq.TQ_PROD, 0, bitmap=bitmap, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE,
                     num_heads=2, seed_sketch=404, calib=calib, device=-1)
    ref = o.spectralquant_codec(calib.float().numpy().astype(np.float64), bitmap, 4, sketch_seed=404)
    assert cb.num_heads == 2 and cb.m == 4
    for h in range(2):
        rot, sk, cen, thr, lv = cb.export(h)
        # Jacobi vs LAPACK on near-degenerate bulk eigenvalues (relative gaps
        # ~1e-6): eigenvectors agree to ~1e-8 absolute, i.e. a few fp32 ulps at most
        assert np.max(np.abs(rot.astype(np.float64) - ref.rot[h])) < 3e-8
        for i in (0, 1, 2, 3, 4, 77, 127):
            Lv = 1 << bitmap[i]
            assert lv[i] == Lv
            # exported fp64 values vs the oracle's fp32-stored ones: within half an fp32 ulp
            assert np.allclose(cen[i, :Lv], ref.centroids[h][i], rtol=7e-8, atol=0)
        assert np.array_equal(sk.astype(np.float32), ref.sketch.astype(np.float32))


@pytest.mark.parametrize("mode,bits,layout", [(tq.TQ_PROD, 3, tq.TQ_LAYOUT_ROW),
                                              (tq.TQ_MSE, 4, tq.TQ_LAYOUT_COL),
                                              (tq.TQ_MSE, 2, tq.TQ_LAYOUT_ROW)])
def test_tile_layout_matches_specification(mode, bits, layout):
    cb = tq.Codebook(128, mode, bits, layout=layout, device=-1)
    ref = o.turboquant_codec(128, bits, "prod" if mode == tq.TQ_PROD else "mse", rot_seed=0,
                             sketch_seed=0, layout="row" if layout == tq.TQ_LAYOUT_ROW else "col")
    assert cb.tile_bytes == o.tile_bytes(ref)
    f = {k: (off, n) for k, off, n in o.tile_fields(ref)}
    assert cb.info.off_nx == f["nx"][0]
    if mode == tq.TQ_PROD:
        assert cb.info.off_nr == f["nr"][0]
    assert cb.records_bytes(100) == 2 * cb.tile_bytes


def test_record_sizes_of_the_workloads():
    k = tq.Codebook(128, tq.TQ_PROD, 3, device=-1)
    v = tq.Codebook(128, tq.TQ_MSE, 4, layout=tq.TQ_LAYOUT_COL, device=-1)
    assert k.tile_bytes == 64 * 52 and v.tile_bytes == 64 * 66
    sq = tq.Codebook(128, tq.TQ_PROD, 0, bitmap=[5, 3, 2, 2] + [1] * 124, qjl_dims=4,
                     rotation=tq.TQ_ROT_GIVEN, num_heads=1, given=np.eye(128), device=-1)
    assert sq.info.code_bytes == 17 and sq.info.sign_bytes == 1 and sq.tile_bytes == 64 * 22


def test_argument_errors_before_launch():
    lib = L.lib()
    with pytest.raises(tq.TQError) as e:
        tq.Codebook(128, tq.TQ_PROD, 1, device=-1)
    assert e.value.status == L.TQ_EINVAL
    with pytest.raises(tq.TQError):
        tq.Codebook(128, 7, 3, device=-1)
    with pytest.raises(tq.TQError) as e:
        tq.Codebook(128, tq.TQ_MSE, 2, bitmap=[2, 1] * 64, layout=tq.TQ_LAYOUT_COL, device=-1)
    assert e.value.status == L.TQ_EUNSUPPORTED
    cb = tq.Codebook(128, tq.TQ_PROD, 3, device=-1)
    buf = ctypes.create_string_buffer(1024)
    # host-only codebook: no device tables -> EINVAL, nothing launched
    st = lib.tq_encode(cb.handle, ctypes.addressof(buf), L.TQ_F32, 1, 1, 4, 0, 0, 128,
                       ctypes.addressof(buf), 0, 0, None, 0, None)
    assert st == L.TQ_EINVAL
    st = lib.tq_encode(cb.handle, None, L.TQ_F32, 1, 1, 4, 0, 0, 128, ctypes.addressof(buf), 0, 0,
                       None, 0, None)
    assert st == L.TQ_EINVAL
    st = lib.tq_encode(cb.handle, ctypes.addressof(buf), 5, 1, 1, 4, 0, 0, 128,
                       ctypes.addressof(buf), 0, 0, None, 0, None)
    assert st == L.TQ_EINVAL
    # tq_encode_kv: tq_encode's checks on both codecs before any launch
    a = ctypes.addressof(buf)
    assert lib.tq_encode_kv(None, cb.handle, a, a, L.TQ_BF16, 1, 1, 4, 0, 0, 128, a, 0, 0, a, 0, 0,
                            None) == L.TQ_EINVAL
    assert lib.tq_encode_kv(cb.handle, cb.handle, a, a, L.TQ_BF16, 1, 1, 4, 0, 0, 128, a, 0, 0, a, 0, 0,
                            None) == L.TQ_EINVAL  # host-only codebooks
    assert lib.tq_encode_kv(cb.handle, cb.handle, a, None, L.TQ_BF16, 1, 1, 4, 0, 0, 128, a, 0, 0, a, 0, 0,
                            None) == L.TQ_EINVAL
    assert lib.tq_encode_kv(cb.handle, cb.handle, a, a, 5, 1, 1, 4, 0, 0, 128, a, 0, 0, a, 0, 0,
                            None) == L.TQ_EINVAL
    assert lib.tq_encode_kv(cb.handle, cb.handle, a, a, L.TQ_BF16, 1, 1, -1, 0, 0, 128, a, 0, 0, a, 0, 0,
                            None) == L.TQ_EINVAL
    assert lib.tq_encode_kv(cb.handle, cb.handle, a, a, L.TQ_BF16, 1, 1, 0, 0, 0, 128, a, 0, 0, a, 0, 0,
                            None) == L.TQ_OK  # nothing to encode
    assert lib.tq_workspace_size(cb.handle, L.TQ_OP_ENCODE, 0, 0, 0) == 0
    wide = tq.Codebook(1536, tq.TQ_PROD, 2, device=-1)
    assert lib.tq_workspace_size(wide.handle, L.TQ_OP_ENCODE, 0, 0, 0) > 0
    assert lib.tq_workspace_size(cb.handle, L.TQ_OP_TOPK, 4, 100, 17) == 0
    assert lib.tq_workspace_size(cb.handle, L.TQ_OP_SCORE, 4, 100, 0) >= 4 * 256 * 4
    assert lib.tq_codebook_free(None) == L.TQ_EINVAL
    assert lib.tq_status_string(L.TQ_EWORKSPACE) == b"workspace too small"
    # device calibration needs a device: refused before any device call
    desc = L.CodebookDesc()
    desc.d, desc.mode, desc.bits, desc.qjl_dims = 128, tq.TQ_PROD, 3, 4
    desc.rotation, desc.num_heads, desc.calib_on_device = tq.TQ_ROT_CALIBRATE, 1, 1
    desc.calib, desc.calib_n, desc.calib_dtype, desc.device = ctypes.addressof(buf), 8, L.TQ_F32, -1
    h = ctypes.c_void_p()
    assert lib.tq_codebook_build(ctypes.byref(desc), ctypes.byref(h)) == L.TQ_EINVAL and not h.value


@pytest.mark.parametrize("mode,bits,heads", [("prod", (3, 2), 1), ("prod", (3, 2), 2), ("mse", (3, 2), 1),
                                             ("prod", (4, 3), 1)])
def test_outlier_split_codebook_matches_oracle(mode, bits, heads):
    # the library's stored-order codec (rotation rows on the channels,
    # block-diagonal sketch, per-dim codebooks) against the oracle's two
    # instances written out in the same order
    rng = np.random.default_rng(heads + bits[0])
    ch = np.stack([rng.permutation(128)[:32] for _ in range(heads)]).astype(np.int32)
    m = tq.TQ_PROD if mode == "prod" else tq.TQ_MSE
    cb = tq.Codebook(128, m, bits[1], seed_rotation=61, seed_sketch=62, outlier_channels=ch,
                     outlier_bits=bits[0], device=-1)
    sc = o.outlier_split_codec(128, ch, bits[0], bits[1], mode, rot_seed=61, sketch_seed=62)
    st = o.split_stored_codec(sc)
    assert cb.num_heads == heads and cb.info.outlier_dims == 32 and cb.info.outlier_per_block == 8
    assert cb.tile_bytes == o.split_tile_bytes(sc)
    fields = dict((f[0], f[1]) for f in o.split_tile_fields(sc))
    assert cb.info.off_nx == fields["nx"] and cb.info.off_nx_o == fields["nx_o"]
    if mode == "prod":
        assert cb.info.off_nr == fields["nr"] and cb.info.off_nr_o == fields["nr_o"]
        assert cb.info.off_signs == fields["sign0"]
    for h in range(heads):
        rot, sk, cen, thr, lv = cb.export(h)
        n, mx = _ulp_mismatch(rot, st.rot[h].astype(np.float32))
        assert mx <= 1 and n <= 4
        assert np.array_equal(lv, 1 << st.bits)
        for i in (0, 7, 8, 31, 32, 127):
            L_ = 1 << int(st.bits[i])
            assert np.allclose(cen[i, :L_], st.centroids[h][i], rtol=0, atol=1e-7)
            assert np.allclose(thr[i, :L_ - 1], st.boundaries[h][i], rtol=0, atol=1e-7)
        if mode == "prod":
            n, mx = _ulp_mismatch(sk, st.sketch.astype(np.float32))
            assert mx <= 1 and n <= 4


def test_outlier_split_argument_errors():
    ch = np.arange(32, dtype=np.int32)
    with pytest.raises(tq.TQError):      # repeated channel
        tq.Codebook(128, tq.TQ_PROD, 2, outlier_channels=np.r_[ch[:31], 0], outlier_bits=3, device=-1)
    with pytest.raises(tq.TQError):      # channel out of range
        tq.Codebook(128, tq.TQ_PROD, 2, outlier_channels=np.r_[ch[:31], 128], outlier_bits=3, device=-1)
    with pytest.raises(tq.TQError):      # o must be 32, 64 or 96
        tq.Codebook(128, tq.TQ_PROD, 2, outlier_channels=ch[:16], outlier_bits=3, device=-1)
    # col records: the 2.5-bit mse split only (32 channels at 3 index bits, the others at 2)
    cb = tq.Codebook(128, tq.TQ_MSE, 2, outlier_channels=ch, outlier_bits=3, layout=tq.TQ_LAYOUT_COL, device=-1)
    assert cb.tile_bytes == 2560  # 8 groups x 288 bytes of code words, two fp16 norms x 64
    for kw in (dict(mode=tq.TQ_PROD, bits=3, outlier_bits=4), dict(mode=tq.TQ_MSE, bits=2, outlier_bits=4),
               dict(mode=tq.TQ_MSE, bits=3, outlier_bits=3)):
        with pytest.raises(tq.TQError):  # other col splits
            tq.Codebook(128, kw["mode"], kw["bits"], outlier_channels=ch, outlier_bits=kw["outlier_bits"],
                        layout=tq.TQ_LAYOUT_COL, device=-1)
    with pytest.raises(tq.TQError):      # col split with 64 outlier channels
        tq.Codebook(128, tq.TQ_MSE, 2, outlier_channels=np.arange(64) * 2, outlier_bits=3,
                    layout=tq.TQ_LAYOUT_COL, device=-1)
    with pytest.raises(tq.TQError):      # d = 128 only
        tq.Codebook(256, tq.TQ_PROD, 2, outlier_channels=ch, outlier_bits=3, device=-1)


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and a message,
    before touching any device."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""
