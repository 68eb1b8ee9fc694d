"""Append-on-decode on the GPU against the CPU oracle: tokens appended one
decode step at a time into existing records must leave exactly the records
the oracle packs for the whole sequences (codes up to the boundary band),
and the decode over them must match (TurboQuant paper review, "Comparison":
tokens generated during decoding are quantized too)."""
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


def _records(codec, cb, encs, cap):
    """Oracle-packed records of each set, zero-padded to cap tokens."""
    per = cb.records_bytes(cap)
    out = []
    for e in encs:
        buf = np.zeros(per, np.uint8)
        if e.idx.shape[0]:
            p = o.pack(codec, e)
            buf[:len(p)] = p
        out.append(buf)
    return np.concatenate(out)


def _take(e, n):
    return o.Encoded(e.idx[:n], None if e.signs is None else e.signs[:n], e.nx[:n],
                     None if e.nr is None else e.nr[:n], e.y[:n], None if e.z is None else e.z[:n])


def _run(kind, dtype=torch.bfloat16):
    B, H, cap, steps = 3, 2, 200, 6
    L0 = [0, 62, 128]
    law = synth.KVLaw(H, 128, 715)
    X = synth.kv_cache(B, H, cap, 128, 711, law).to(dtype)  # token t of (b, h) = X[b, h, t]
    if kind == "sq":
        calib = torch.stack([law.sample(h, 1024, torch.Generator().manual_seed(705 + h), "cpu") for h in range(H)])
        bitmap = [5, 3, 2, 2] + [1] * 124
        cb = tq.Codebook(128, tq.TQ_PROD, 0, bitmap=bitmap, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE,
                         num_heads=H, seed_sketch=704, calib=calib)
        codec = o.spectralquant_codec(calib.float().numpy().astype(np.float64), bitmap, 4, sketch_seed=704)
    elif kind == "values":
        cb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=707, layout=tq.TQ_LAYOUT_COL)
        codec = o.turboquant_codec(128, 4, "mse", rot_seed=707, layout="col")
    elif kind == "values_hadamard":
        cb = tq.Codebook(128, tq.TQ_MSE, 4, rotation=tq.TQ_ROT_HADAMARD, seed_rotation=707, layout=tq.TQ_LAYOUT_COL)
        codec = o.turboquant_codec(128, 4, "mse", rot_seed=707, layout="col", rotation="hadamard")
    elif kind == "values2":
        cb = tq.Codebook(128, tq.TQ_MSE, 2, seed_rotation=707, layout=tq.TQ_LAYOUT_COL)
        codec = o.turboquant_codec(128, 2, "mse", rot_seed=707, layout="col")
    else:
        rot = tq.TQ_ROT_HADAMARD if kind == "keys_hadamard" else tq.TQ_ROT_HAAR
        cb = tq.Codebook(128, tq.TQ_PROD, 3, rotation=rot, seed_rotation=703, seed_sketch=704)
        codec = o.turboquant_codec(128, 3, "prod", rot_seed=703, sketch_seed=704,
                                   rotation="hadamard" if kind == "keys_hadamard" else "haar")
    heads = H if kind == "sq" else 1
    full = {(b, h): o.encode(codec, X[b, h].double().numpy(), head=h if heads > 1 else 0)
            for b in range(B) for h in range(H)}
    init = [_take(full[b, h], L0[b]) for b in range(B) for h in range(H)]
    rec = torch.from_numpy(_records(codec, cb, init, cap)).to(DEV)
    for s in range(steps):
        pos = torch.tensor([L0[b] + s for b in range(B)], dtype=torch.int32, device=DEV)
        xs = torch.stack([X[b, :, L0[b] + s] for b in range(B)]).to(DEV)  # [B][H][d]
        tq.append(cb, xs, rec, pos, cap)
    # a position past the capacity writes nothing
    tq.append(cb, xs, rec, torch.tensor([cap] * B, dtype=torch.int32, device=DEV), cap)
    got_all = rec.cpu().numpy()
    per = cb.records_bytes(cap)
    for b in range(B):
        for h in range(H):
            n = L0[b] + steps
            buf = got_all[(b * H + h) * per:(b * H + h + 1) * per]
            got = o.unpack(codec, buf, n)
            st = check_encoded(codec, _take(full[b, h], n), got, head=h if heads > 1 else 0)
            # nothing outside the n written tokens
            want = np.zeros(per, np.uint8)
            p = o.pack(codec, got)
            want[:len(p)] = p
            assert np.array_equal(buf, want)
            say(kind, b, h, st)
    return cb, codec, rec, full, L0, steps, X


@pytest.mark.parametrize("kind", ["keys", "values", "values2", "sq", "keys_hadamard", "values_hadamard"])
def test_append_matches_whole_sequence_encode(kind):
    _run(kind)


def test_append_fp32_input():
    _run("keys", dtype=torch.float32)


@pytest.mark.parametrize("kind", ["keys", "values"])
def test_append_special_rows(kind):
    """One appended vector per head: zeros, -0, magnitudes near 1e-30 (whose
    squares underflow fp32), one nonzero coordinate, near 1e3, and a Gaussian
    row (bf16), into slot 0; against the oracle's encode of the same rows."""
    H = 6
    g = torch.Generator().manual_seed(47)
    x = torch.randn(H, 128, generator=g)
    x[0] = 0.0
    x[1] = -torch.zeros(128)
    x[2] *= 1e-30
    x[3] = 0.0
    x[3, 77] = -1.5
    x[4] *= 1e3
    xb = x.to(torch.bfloat16)
    if kind == "keys":
        cb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=31, seed_sketch=32)
        codec = o.turboquant_codec(128, 3, "prod", rot_seed=31, sketch_seed=32)
    else:
        cb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=31, layout=tq.TQ_LAYOUT_COL)
        codec = o.turboquant_codec(128, 4, "mse", rot_seed=31, layout="col")
    cap = 64
    per = cb.records_bytes(cap)
    rec = torch.zeros(H * per, dtype=torch.uint8, device=DEV)
    tq.append(cb, xb.reshape(1, H, 128).to(DEV), rec, torch.zeros(1, dtype=torch.int32, device=DEV), cap)
    torch.cuda.synchronize()
    buf = rec.cpu().numpy()
    ref = o.encode(codec, xb.double().numpy())
    heads = [o.unpack(codec, buf[h * per:(h + 1) * per], cap) for h in range(H)]
    got = o.Encoded(np.stack([e.idx[0] for e in heads]),
                    None if ref.signs is None else np.stack([e.signs[0] for e in heads]),
                    np.array([e.nx[0] for e in heads]),
                    None if ref.nr is None else np.array([e.nr[0] for e in heads]), None, None)
    say(kind, check_encoded(codec, ref, got))
    assert float(got.nx[0]) == 0.0 and float(got.nx[1]) == 0.0


def test_decode_after_append():
    kcb, kc, krec, kfull, L0, steps, K = _run("keys")
    vcb, vc, vrec, vfull, _, _, V = _run("values")
    B, H, Hq = 3, 2, 8
    law = synth.KVLaw(H, 128, 715)
    q = synth.kv_queries(B, Hq, H, 128, 712, law)
    lens = [L0[b] + steps for b in range(B)]
    scale = 1 / math.sqrt(128)
    ref = np.stack([o.decode_attention(kc, vc, q[b].double().numpy(), [_take(kfull[b, h], lens[b]) for h in range(H)],
                                       [_take(vfull[b, h], lens[b]) for h in range(H)], scale) for b in range(B)])
    out = tq.decode_attend(kcb, vcb, q.to(DEV), krec, vrec, 200, H, scale,
                           seq_lens=torch.tensor(lens, dtype=torch.int32, device=DEV)).cpu().numpy()
    nvmax = max(float(np.max(vfull[b, h].nx.astype(np.float64))) for b in range(B) for h in range(H))
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"decode after append: max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3
