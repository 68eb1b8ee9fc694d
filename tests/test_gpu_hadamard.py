"""Parity of the randomized Hadamard rotation mode on the GPU against the
CPU oracle (launch post of the reference cache: its O(d log d) rotation
mode), whose Pi is the dense matrix H diag(s) / sqrt(d).  On the GPU the
d = 128 bf16 encode of the GQA K/V codecs runs the register Walsh-Hadamard
kernel, the query rotation of score / top-k / decode, the inverse value
rotation of decode and the append run the wave transform; the other encodes
use the materialised Pi."""
import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_compression_encode_amd as tq
import synth
from oracle import tq_oracle as o
from tests.parity import check_encoded, check_scores

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
HAD = tq.TQ_ROT_HADAMARD


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def up(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def _codecs(rseed, sseed):
    kcb = tq.Codebook(128, tq.TQ_PROD, 3, rotation=HAD, seed_rotation=rseed, seed_sketch=sseed)
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, rotation=HAD, seed_rotation=rseed, layout=tq.TQ_LAYOUT_COL)
    kc = o.turboquant_codec(128, 3, "prod", rot_seed=rseed, sketch_seed=sseed, rotation="hadamard")
    vc = o.turboquant_codec(128, 4, "mse", rot_seed=rseed, layout="col", rotation="hadamard")
    return kcb, vcb, kc, vc


@pytest.mark.parametrize("T", [1000, 1, 64, 4096])
def test_encode_kv_bf16_hadamard(T):
    say(f"hadamard kv encode bf16 T={T}")
    H = 2
    law = synth.KVLaw(H, 128, synth.seed(2, "calibration"))
    k = synth.kv_cache(1, H, T, 128, 211, law)[0]
    v = synth.kv_cache(1, H, T, 128, 261, law)[0]
    kcb, vcb, kc, vc = _codecs(213, 214)
    kb = tq.encode(kcb, k.to(DEV)).cpu().numpy()
    vb = tq.encode(vcb, v.to(DEV)).cpu().numpy()
    per_k, per_v = kcb.records_bytes(T), vcb.records_bytes(T)
    for h in range(H):
        rk = o.encode(kc, k[h].double().numpy())
        rv = o.encode(vc, v[h].double().numpy())
        gk = o.unpack(kc, kb[h * per_k:(h + 1) * per_k], T)
        gv = o.unpack(vc, vb[h * per_v:(h + 1) * per_v], T)
        say("K", check_encoded(kc, rk, gk))
        say("V", check_encoded(vc, rv, gv))
        # slots past T in the last tile are zero
        assert np.array_equal(o.pack(kc, gk), kb[h * per_k:(h + 1) * per_k])
        assert np.array_equal(o.pack(vc, gv), vb[h * per_v:(h + 1) * per_v])


def test_encode_hadamard_zero_vectors():
    x = torch.zeros(70, 128, dtype=torch.bfloat16)
    x[3] = 1.0
    kcb, vcb, kc, vc = _codecs(5, 6)
    for cb, codec in ((kcb, kc), (vcb, vc)):
        buf = tq.encode(cb, x.to(DEV)).cpu().numpy()
        say(check_encoded(codec, o.encode(codec, x.double().numpy()), o.unpack(codec, buf, 70)))


@pytest.mark.parametrize("bits,mode,layout,dtype", [(3, tq.TQ_PROD, tq.TQ_LAYOUT_ROW, torch.float32),
                                                    (2, tq.TQ_MSE, tq.TQ_LAYOUT_ROW, torch.bfloat16),
                                                    (4, tq.TQ_PROD, tq.TQ_LAYOUT_ROW, torch.bfloat16)])
def test_encode_hadamard_dense_path(bits, mode, layout, dtype):
    # combinations outside the register transform use the materialised Pi
    n = 777
    say(f"hadamard dense-path encode bits={bits} mode={mode} dtype={dtype}")
    x = synth.iid_gaussian(n, 128, 17).to(dtype)
    cb = tq.Codebook(128, mode, bits, rotation=HAD, seed_rotation=31, seed_sketch=32, layout=layout)
    codec = o.turboquant_codec(128, bits, "prod" if mode == tq.TQ_PROD else "mse", rot_seed=31,
                               sketch_seed=32, rotation="hadamard")
    buf = tq.encode(cb, x.to(DEV)).cpu().numpy()
    say(check_encoded(codec, o.encode(codec, x.double().numpy()), o.unpack(codec, buf, n)))


@pytest.mark.parametrize("bits", [3, 4])
def test_score_hadamard(bits):
    # query rotation by the wave transform (prod: then the dense sketch)
    say(f"hadamard score bits={bits}")
    n = 3000
    x = synth.iid_gaussian(n, 128, 41)
    q = synth.iid_gaussian(16, 128, 42)
    cb = tq.Codebook(128, tq.TQ_PROD, bits, rotation=HAD, seed_rotation=43, seed_sketch=44)
    codec = o.turboquant_codec(128, bits, "prod", rot_seed=43, sketch_seed=44, rotation="hadamard")
    ref = o.encode(codec, x.double().numpy())
    s = tq.score(cb, q.to(DEV), up(o.pack(codec, ref)), n).cpu().numpy()
    say("max scaled error", check_scores(s, o.score(codec, q.double().numpy(), ref), q.numpy(), ref.nx))
    cbm = tq.Codebook(128, tq.TQ_MSE, bits, rotation=HAD, seed_rotation=43)
    cm = o.turboquant_codec(128, bits, "mse", rot_seed=43, rotation="hadamard")
    rm = o.encode(cm, x.double().numpy())
    s = tq.score(cbm, q.to(DEV), up(o.pack(cm, rm)), n).cpu().numpy()
    say("mse max scaled error", check_scores(s, o.score(cm, q.double().numpy(), rm), q.numpy(), rm.nx))


def test_search_topk_hadamard():
    n, d, nq, k = 20000, 128, 8, 10
    x = synth.iid_gaussian(n, d, 45)
    q = synth.iid_gaussian(nq, d, 46)
    cb = tq.Codebook(d, tq.TQ_PROD, 2, rotation=HAD, seed_rotation=47, seed_sketch=48)
    codec = o.turboquant_codec(d, 2, "prod", rot_seed=47, sketch_seed=48, rotation="hadamard")
    ref = o.encode(codec, x.double().numpy())
    s, i = tq.search_topk(cb, q.to(DEV), up(o.pack(codec, ref)), n, k)
    s, i = s.cpu().numpy(), i.cpu().numpy()
    full = o.score(codec, q.double().numpy(), ref)
    rs, ri = o.topk(full, k)
    for r in range(nq):
        tol = 1e-3 * np.linalg.norm(q[r].numpy()) * ref.nx.astype(np.float64)
        kth = rs[r, -1]
        diff = set(i[r].tolist()) ^ set(ri[r].tolist())
        assert all(abs(full[r, j] - kth) <= 2 * tol[j] for j in diff), f"query {r}: top-k differs beyond near-ties"
        assert np.all(np.abs(s[r] - full[r, i[r]]) <= tol[i[r]])


@pytest.mark.parametrize("T,key_bits", [(700, 3), (300, 3), (700, 4)])
def test_decode_attend_hadamard(T, key_bits):
    # T = 700: several splits, merged by the combine kernel (inverse value
    # rotation there); T = 300: one split, rotated back inside the MFMA
    # kernel; 4-bit keys: the generic kernel after the query-prep kernel
    say(f"hadamard decode T={T} key bits={key_bits}")
    B, Hq, Hkv = 2, 8, 2
    law = synth.KVLaw(Hkv, 128, 225)
    K = synth.kv_cache(B, Hkv, T, 128, 221, law)
    V = synth.kv_cache(B, Hkv, T, 128, 271, law)
    q = synth.kv_queries(B, Hq, Hkv, 128, 222, law)
    kcb, vcb, kc, vc = _codecs(223, 224)
    if key_bits != 3:
        kcb = tq.Codebook(128, tq.TQ_PROD, key_bits, rotation=HAD, seed_rotation=223, seed_sketch=224)
        kc = o.turboquant_codec(128, key_bits, "prod", rot_seed=223, sketch_seed=224, rotation="hadamard")
    ke = [[o.encode(kc, K[b, g].double().numpy()) for g in range(Hkv)] for b in range(B)]
    ve = [[o.encode(vc, V[b, g].double().numpy()) for g in range(Hkv)] for b in range(B)]
    kbuf = np.concatenate([o.pack(kc, e) for row in ke for e in row])
    vbuf = np.concatenate([o.pack(vc, e) for row in ve for e in row])
    scale = 1 / math.sqrt(128)
    ref = np.stack([o.decode_attention(kc, vc, q[b].double().numpy(), ke[b], ve[b], scale) for b in range(B)])
    out = tq.decode_attend(kcb, vcb, q.to(DEV), up(kbuf), up(vbuf), T, Hkv, scale).cpu().numpy()
    nvmax = max(float(np.max(e.nx.astype(np.float64))) for row in ve for e in row)
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"hadamard decode: max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3
