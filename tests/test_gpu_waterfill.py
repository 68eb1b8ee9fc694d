"""SpectralQuant with the bit map water-filled from the calibration spectrum
(SpectralQuant thread, tweet 6) on the GPU against the CPU oracle: the codec
is built from the same calibration keys on both sides, then encode and the
fused decode are compared."""
import math
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def up(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def _codecs(law, hkv, budget):
    calib = torch.stack([law.sample(h, 2048, torch.Generator().manual_seed(605 + h), "cpu") for h in range(hkv)])
    kcb = tq.Codebook(128, tq.TQ_PROD, 0, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE, num_heads=hkv,
                      seed_sketch=604, calib=calib, waterfill_bits=budget)
    kc = o.spectralquant_codec(calib.float().numpy().astype(np.float64), None, 4, sketch_seed=604,
                               waterfill_bits=budget)
    return kcb, kc


@pytest.mark.parametrize("budget", [136, 140])
def test_waterfill_encode_and_decode(budget):
    B, Hq, Hkv, T = 2, 8, 2, 600
    law = synth.KVLaw(Hkv, 128, 615)
    kcb, kc = _codecs(law, Hkv, budget)
    say(f"water-filled bits (budget {budget}):", kc.bits[:8].tolist(), "... sum", int(kc.bits.sum()))
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=607, layout=tq.TQ_LAYOUT_COL)
    vc = o.turboquant_codec(128, 4, "mse", rot_seed=607, layout="col")
    K = synth.kv_cache(B, Hkv, T, 128, 611, law)
    V = synth.kv_cache(B, Hkv, T, 128, 651, law)
    q = synth.kv_queries(B, Hq, Hkv, 128, 612, law)
    # encode parity, per head (each head has its own eigenbasis)
    kb = tq.encode(kcb, K.to(DEV)).cpu().numpy()
    per = kcb.records_bytes(T)
    for b in range(B):
        for g in range(Hkv):
            ref = o.encode(kc, K[b, g].double().numpy(), head=g)
            got = o.unpack(kc, kb[(b * Hkv + g) * per:(b * Hkv + g + 1) * per], T)
            say("K", b, g, check_encoded(kc, ref, got, head=g))
    # decode on oracle-packed records
    ke = [[o.encode(kc, K[b, g].double().numpy(), head=g) for g in range(Hkv)] for b in range(B)]
    ve = [[o.encode(vc, V[b, g].double().numpy()) for g in range(Hkv)] for b in range(B)]
    kbuf = np.concatenate([o.pack(kc, e) for row in ke for e in row])
    vbuf = np.concatenate([o.pack(vc, e) for row in ve for e in row])
    scale = 1 / math.sqrt(128)
    ref = np.stack([o.decode_attention(kc, vc, q[b].double().numpy(), ke[b], ve[b], scale) for b in range(B)])
    out = tq.decode_attend(kcb, vcb, q.to(DEV), up(kbuf), up(vbuf), T, Hkv, scale).cpu().numpy()
    nvmax = max(float(np.max(e.nx.astype(np.float64))) for row in ve for e in row)
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"water-filled decode: max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3
