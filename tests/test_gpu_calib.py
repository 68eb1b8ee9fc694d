"""SpectralQuant calibration with its moments formed on the GPU ([SQ] tweet 4:
the per-head eigenbasis from a short calibration pass).  The codebook built
from device-resident calibration vectors must match the CPU oracle's
calibration (eigenbasis, per-dim scales and levels, water-filled bit map),
and the keys it encodes must match the oracle's encode with the oracle's own
calibration."""
import sys

import numpy as np
import pytest
import torch

import kv_cache_compression_encode_amd as tq
import synth
from oracle import tq_oracle as o
from tests.parity import check_encoded

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BITMAP = [5, 3, 2, 2] + [1] * 124


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _calib(law, heads, n, seed, dtype):
    return torch.stack([law.sample(h, n, torch.Generator().manual_seed(seed + h), "cpu")
                        for h in range(heads)]).to(dtype)


@pytest.mark.parametrize("dtype,n", [(torch.bfloat16, 2048), (torch.float32, 1000)])
def test_device_calibration_matches_oracle(dtype, n):
    # n = 1000: a ragged last stage of the moment kernel (1000 = 31 x 32 + 8)
    say(f"device calibration dtype={dtype} n={n}")
    H = 2
    law = synth.KVLaw(H, 128, 405)
    calib = _calib(law, H, n, 407, dtype)
    cb = tq.Codebook(128, tq.TQ_PROD, 0, bitmap=BITMAP, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE,
                     num_heads=H, seed_sketch=404, calib=calib.to(DEV))
    ref = o.spectralquant_codec(calib.float().numpy().astype(np.float64), BITMAP, 4, sketch_seed=404)
    for h in range(H):
        rot, sk, cen, thr, lv = cb.export(h)
        # Jacobi on the fp64 device moments vs LAPACK on the oracle's
        # covariance: near-degenerate bulk eigenvalues leave ~1e-8 differences
        err = np.max(np.abs(rot.astype(np.float64) - ref.rot[h]))
        say(f"head {h}: max |Pi - Pi_oracle| = {err:.3g}")
        assert err < 3e-8
        for i in range(128):
            Lv = 1 << BITMAP[i]
            assert lv[i] == Lv
            assert np.allclose(cen[i, :Lv], ref.centroids[h][i], rtol=1e-7, atol=0)


def test_device_calibration_matches_host_build():
    # the same vectors through the host and the device calibration
    H = 3
    law = synth.KVLaw(H, 128, 415)
    calib = _calib(law, H, 2048, 417, torch.bfloat16)
    kw = dict(bitmap=BITMAP, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE, num_heads=H, seed_sketch=404)
    dev = tq.Codebook(128, tq.TQ_PROD, 0, calib=calib.to(DEV), **kw)
    host = tq.Codebook(128, tq.TQ_PROD, 0, calib=calib, **kw)
    for h in range(H):
        rd, _, cd, td, _ = dev.export(h)
        rh, _, ch, th, _ = host.export(h)
        assert np.max(np.abs(rd.astype(np.float64) - rh)) < 3e-8
        assert np.allclose(cd, ch, rtol=1e-6, atol=0)


def test_device_calibration_waterfill_and_encode():
    H, T = 2, 700
    law = synth.KVLaw(H, 128, 425)
    calib = _calib(law, H, 2048, 427, torch.bfloat16)
    kcb = tq.Codebook(128, tq.TQ_PROD, 0, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE, num_heads=H,
                      seed_sketch=404, calib=calib.to(DEV), waterfill_bits=136)
    kc = o.spectralquant_codec(calib.float().numpy().astype(np.float64), None, 4, sketch_seed=404,
                               waterfill_bits=136)
    lv = kcb.export(0)[4]
    assert np.array_equal(lv, 1 << kc.bits), (lv[:8], kc.bits[:8])
    K = synth.kv_cache(1, H, T, 128, 421, law)[0]
    buf = tq.encode(kcb, K.to(DEV)).cpu().numpy()
    per = kcb.records_bytes(T)
    for h in range(H):
        ref = o.encode(kc, K[h].double().numpy(), head=h)
        say("SQ K (device calibration)", check_encoded(kc, ref, o.unpack(kc, buf[h * per:(h + 1) * per], T), head=h))
