"""Parity of the HIP path against the CPU oracle on seeded synthetic inputs
(MI355X).  Every call goes through the C ABI via the thin binding."""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def up(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def gpu_records(cb, x, **kw):
    rec = tq.encode(cb, x.to(DEV), **kw)
    torch.cuda.synchronize()
    return rec.cpu().numpy()


def test_encode_many_sets():
    # 2 x 32800 (sequence, head) sets of one token: more than 65535 sets, so
    # the grid continues along z; sampled sets against the oracle
    B, H = 2, 32800
    say(f"encode {B} x {H} sets of one token")
    x = synth.iid_gaussian(B * H, 128, 31).reshape(B, H, 1, 128).to(torch.bfloat16)
    cb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=33, seed_sketch=34)
    codec = o.turboquant_codec(128, 3, "prod", rot_seed=33, sketch_seed=34)
    buf = gpu_records(cb, x)
    per = cb.records_bytes(1)
    assert buf.shape[0] == B * H * per
    for bh in (0, 1, 65534, 65535, 65536, B * H - 1):
        b, h = divmod(bh, H)
        ref = o.encode(codec, x[b, h].double().numpy())
        got = o.unpack(codec, buf[bh * per:(bh + 1) * per], 1)
        check_encoded(codec, ref, got)
        assert np.array_equal(o.pack(codec, got), buf[bh * per:(bh + 1) * per])


# ------------------------------------------------ plain TurboQuant-prod, d=128
@pytest.mark.parametrize("n", [4096, 1, 63, 65, 1000])
def test_encode_prod_fp32_d128(n):
    say(f"encode prod b=3 fp32 n={n}")
    x = synth.iid_gaussian(n, 128, synth.seed(1, "data"))
    cb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=103, seed_sketch=104)
    codec = o.turboquant_codec(128, 3, "prod", rot_seed=103, sketch_seed=104)
    buf = gpu_records(cb, x)
    assert len(buf) == cb.records_bytes(n)
    ref = o.encode(codec, x.double().numpy())
    got = o.unpack(codec, buf, n)
    say(check_encoded(codec, ref, got))
    # slots past n in the last tile are zero
    assert np.array_equal(o.pack(codec, got), buf)


def test_score_prod_d128():
    say("score 16 x 4096")
    x = synth.iid_gaussian(4096, 128, synth.seed(1, "data"))
    q = synth.iid_gaussian(16, 128, synth.seed(1, "queries"))
    cb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=103, seed_sketch=104)
    codec = o.turboquant_codec(128, 3, "prod", rot_seed=103, sketch_seed=104)
    ref = o.encode(codec, x.double().numpy())
    s = tq.score(cb, q.to(DEV), up(o.pack(codec, ref)), 4096).cpu().numpy()
    r = check_scores(s, o.score(codec, q.double().numpy(), ref), q.numpy(), ref.nx)
    say("max scaled error", r)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_encode_mse_row_bf16(bits):
    """TurboQuant-mse with row records from bf16 KV rows (the row-layout value
    encode), 777 vectors over two heads' worth of tiles, against the oracle."""
    n = 777
    law = synth.KVLaw(1, 128, 61)
    x = synth.kv_cache(1, 1, n, 128, 62, law)[0, 0]
    cb = tq.Codebook(128, tq.TQ_MSE, bits, seed_rotation=63)
    codec = o.turboquant_codec(128, bits, "mse", rot_seed=63)
    ref = o.encode(codec, x.double().numpy())
    got = o.unpack(codec, gpu_records(cb, x), n)
    say(bits, check_encoded(codec, ref, got))


@pytest.mark.parametrize("bits,mode", [(2, tq.TQ_MSE), (4, tq.TQ_MSE), (2, tq.TQ_PROD), (5, tq.TQ_PROD)])
def test_encode_and_score_other_bits(bits, mode):
    say(f"bits={bits} mode={mode}")
    n = 777
    x = synth.iid_gaussian(n, 128, 7)
    q = synth.iid_gaussian(5, 128, 8)
    mname = "prod" if mode == tq.TQ_PROD else "mse"
    cb = tq.Codebook(128, mode, bits, seed_rotation=9, seed_sketch=10)
    codec = o.turboquant_codec(128, bits, mname, rot_seed=9, sketch_seed=10)
    ref = o.encode(codec, x.double().numpy())
    say(check_encoded(codec, ref, o.unpack(codec, gpu_records(cb, x), n)))
    s = tq.score(cb, q.to(DEV), up(o.pack(codec, ref)), n).cpu().numpy()
    check_scores(s, o.score(codec, q.double().numpy(), ref), q.numpy(), ref.nx)


def test_zero_vectors_and_empty():
    cb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=1, seed_sketch=2)
    codec = o.turboquant_codec(128, 3, "prod", rot_seed=1, sketch_seed=2)
    x = torch.zeros(70, 128)
    x[5] = 1.0
    buf = gpu_records(cb, x)
    got = o.unpack(codec, buf, 70)
    ref = o.encode(codec, x.double().numpy())
    assert float(got.nx[0]) == 0.0
    # y = 0 lies on the middle boundary: codes there are in the band by rule;
    # the stored record must still score exactly 0
    s = tq.score(cb, torch.ones(1, 128, device=DEV), torch.from_numpy(buf).to(DEV), 70).cpu().numpy()
    assert s[0, 0] == 0.0
    assert np.all(got.nx[[i for i in range(70) if i != 5]] == 0)
    out = tq.encode(cb, torch.zeros(0, 128, device=DEV), records=torch.zeros(16, dtype=torch.uint8, device=DEV))
    assert out.shape[0] == 16


@pytest.mark.parametrize("kind", ["keys", "values", "keys_fp32", "keys_hadamard", "values_hadamard"])
def test_bf16_special_rows(kind):
    """Rows that are all +0, all -0, one nonzero coordinate, signed zeros
    among nonzeros, and magnitudes near 1e-30 (whose squares underflow fp32:
    the encoders' scaled norm path) and 1e3, among Gaussian rows, 100 rows
    (one full tile and a ragged one), bf16 (fp32 for keys_fp32), dense or
    Hadamard rotation: codes, signs and norms against the oracle under the
    usual rules; the all-zero rows store n_x = 0 and, for keys, the signs of
    S(0 - c)."""
    n = 100
    g = torch.Generator().manual_seed(41)
    x = torch.randn(n, 128, generator=g)
    x[3] = 0.0
    x[4] = -torch.zeros(128)
    x[5] = 0.0
    x[5, 17] = -2.5
    x[6, ::2] = -0.0
    x[7, 1::3] = 0.0
    x[8] *= 1e-30
    x[9] *= 1e3
    x[70] = -torch.zeros(128)
    xb = x if kind == "keys_fp32" else x.to(torch.bfloat16)
    rot = {"rotation": tq.TQ_ROT_HADAMARD} if kind.endswith("hadamard") else {}
    orot = {"rotation": "hadamard"} if kind.endswith("hadamard") else {}
    if kind.startswith("keys"):
        cb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=21, seed_sketch=22, **rot)
        codec = o.turboquant_codec(128, 3, "prod", rot_seed=21, sketch_seed=22, **orot)
    else:
        cb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=21, layout=tq.TQ_LAYOUT_COL, **rot)
        codec = o.turboquant_codec(128, 4, "mse", rot_seed=21, layout="col", **orot)
    ref = o.encode(codec, xb.double().numpy())
    got = o.unpack(codec, gpu_records(cb, xb), n)
    say(kind, check_encoded(codec, ref, got))
    for r in (3, 4, 70):
        assert float(got.nx[r]) == 0.0
        if kind.startswith("keys"):
            assert np.array_equal(got.signs[r], ref.signs[r])
    assert float(got.nx[8]) == float(ref.nx[8])


# --------------------------------------------------------- bf16 KV workload
def kv_inputs(heads, tokens, seed):
    law = synth.KVLaw(heads, 128, synth.seed(2, "calibration"))
    k = synth.kv_cache(1, heads, tokens, 128, seed, law)[0]
    v = synth.kv_cache(1, heads, tokens, 128, seed + 50, law)[0]
    return law, k, v


def test_encode_kv_bf16():
    say("kv encode bf16 K prod b=3 row, V mse b=4 col")
    H, T = 2, 1000
    law, k, v = kv_inputs(H, T, synth.seed(2, "data"))
    kcb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=203, seed_sketch=204)
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=203, layout=tq.TQ_LAYOUT_COL)
    kc = o.turboquant_codec(128, 3, "prod", rot_seed=203, sketch_seed=204)
    vc = o.turboquant_codec(128, 4, "mse", rot_seed=203, layout="col")
    kb, vb = gpu_records(kcb, k), gpu_records(vcb, v)
    per_k, per_v = kcb.records_bytes(T), vcb.records_bytes(T)
    for h in range(H):
        rk = o.encode(kc, k[h].double().numpy())
        rv = o.encode(vc, v[h].double().numpy())
        say("K", check_encoded(kc, rk, o.unpack(kc, kb[h * per_k:(h + 1) * per_k], T)))
        say("V", check_encoded(vc, rv, o.unpack(vc, vb[h * per_v:(h + 1) * per_v], T)))


def _decode_case(B, Hq, Hkv, T, seq_lens=None, sq=False):
    law = synth.KVLaw(Hkv, 128, 205)
    K = synth.kv_cache(B, Hkv, T, 128, 201, law)
    V = synth.kv_cache(B, Hkv, T, 128, 251, law)
    q = synth.kv_queries(B, Hq, Hkv, 128, 202, law)
    if sq:
        calib = torch.stack([law.sample(h, 2048, torch.Generator().manual_seed(405 + h), "cpu")
                             for h in range(Hkv)])
        bitmap = [5, 3, 2, 2] + [1] * 124
        kcb = tq.Codebook(128, tq.TQ_PROD, 0, bitmap=bitmap, qjl_dims=4,
                          rotation=tq.TQ_ROT_CALIBRATE, num_heads=Hkv, seed_sketch=404, calib=calib)
        kc = o.spectralquant_codec(calib.float().numpy().astype(np.float64), bitmap, 4, sketch_seed=404)
    else:
        kcb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=203, seed_sketch=204)
        kc = o.turboquant_codec(128, 3, "prod", rot_seed=203, sketch_seed=204)
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=207, layout=tq.TQ_LAYOUT_COL)
    vc = o.turboquant_codec(128, 4, "mse", rot_seed=207, layout="col")
    kbuf, vbuf, outs = [], [], []
    ke_all, ve_all = [], []
    for b in range(B):
        ke = [o.encode(kc, K[b, g].double().numpy(), head=g if sq else 0) for g in range(Hkv)]
        ve = [o.encode(vc, V[b, g].double().numpy()) for g in range(Hkv)]
        ke_all.append(ke)
        ve_all.append(ve)
        kbuf += [o.pack(kc, e) for e in ke]
        vbuf += [o.pack(vc, e) for e in ve]
    scale = 1 / math.sqrt(128)
    lens = seq_lens if seq_lens is not None else [T] * B
    ref = np.zeros((B, Hq, 128))
    for b in range(B):
        L_ = lens[b]
        kk = [o.Encoded(e.idx[:L_], None if e.signs is None else e.signs[:L_], e.nx[:L_],
                        None if e.nr is None else e.nr[:L_], None, None) for e in ke_all[b]]
        vv = [o.Encoded(e.idx[:L_], None, e.nx[:L_], None, None, None) for e in ve_all[b]]
        if L_ > 0:
            ref[b] = o.decode_attention(kc, vc, q[b].double().numpy(), kk, vv, scale)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV) if seq_lens is not None else None
    out = tq.decode_attend(kcb, vcb, q.to(DEV), up(np.concatenate(kbuf)), up(np.concatenate(vbuf)),
                           T, Hkv, scale, seq_lens=sl).cpu().numpy()
    nvmax = max(float(np.max(e.nx.astype(np.float64))) for ve in ve_all for e in ve)
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"decode B={B} Hq={Hq} Hkv={Hkv} T={T} sq={sq}: max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3


def test_decode_attend_small():
    _decode_case(1, 8, 2, 1000)


def test_decode_attend_gqa_batch_and_seq_lens():
    _decode_case(3, 16, 4, 300, seq_lens=[300, 1, 129])


def test_decode_attend_empty_sequences():
    # a sequence with no tokens attends to nothing: its output is zero (also
    # when several splits see no tile); the others are unaffected
    _decode_case(4, 8, 2, 700, seq_lens=[0, 700, 0, 65])


def test_decode_attend_max_tokens_zero():
    # an empty cache: all outputs zero, and no record is read (the record
    # buffers here hold a single byte)
    kcb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=203, seed_sketch=204)
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=207, layout=tq.TQ_LAYOUT_COL)
    q = torch.randn(2, 8, 128, device=DEV)
    rec = torch.zeros(16, dtype=torch.uint8, device=DEV)
    out = torch.full((2, 8, 128), 7.0, device=DEV)
    tq.decode_attend(kcb, vcb, q, rec, rec, 0, 2, 0.1, out=out)
    sl = torch.zeros(2, dtype=torch.int32, device=DEV)
    tq.decode_attend(kcb, vcb, q, rec, rec, 0, 2, 0.1, seq_lens=sl)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_decode_attend_spectralquant():
    _decode_case(2, 8, 2, 500, sq=True)


def test_decode_attend_many_splits():
    # one sequence and one KV head over 70000 tokens: 137 splits of 8 tiles,
    # more than the merge kernel takes in one round of loads
    _decode_case(1, 4, 1, 70000, seq_lens=[70000 - 37])


def test_encode_spectralquant():
    Hkv, T = 2, 700
    law = synth.KVLaw(Hkv, 128, 405)
    K = synth.kv_cache(1, Hkv, T, 128, 401, law)[0]
    calib = torch.stack([law.sample(h, 2048, torch.Generator().manual_seed(405 + h), "cpu")
                         for h in range(Hkv)])
    bitmap = [5, 3, 2, 2] + [1] * 124
    kcb = tq.Codebook(128, tq.TQ_PROD, 0, bitmap=bitmap, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE,
                      num_heads=Hkv, seed_sketch=404, calib=calib)
    kc = o.spectralquant_codec(calib.float().numpy().astype(np.float64), bitmap, 4, sketch_seed=404)
    buf = gpu_records(kcb, K)
    per = kcb.records_bytes(T)
    for h in range(Hkv):
        ref = o.encode(kc, K[h].double().numpy(), head=h)
        say("SQ K", check_encoded(kc, ref, o.unpack(kc, buf[h * per:(h + 1) * per], T), head=h))


# ------------------------------------------------------------------- top-k
@pytest.mark.parametrize("mode,bits,k", [("prod", 2, 10), ("prod", 3, 16), ("prod", 4, 1), ("mse", 2, 7),
                                         ("mse", 3, 12)])
def test_search_topk_small(mode, bits, k):
    # 1, 2 and 3 index bits (the MFMA search), both list sizes (k <= 10 and
    # k <= 16), prod and mse; 20000 keys over several workgroup splits
    n, d, nq = 20000, 128, 8
    x = synth.iid_gaussian(n, d, 501)
    x = x / x.norm(dim=1, keepdim=True)
    q = synth.iid_gaussian(nq, d, 502)
    m = tq.TQ_PROD if mode == "prod" else tq.TQ_MSE
    cb = tq.Codebook(d, m, bits, seed_rotation=503, seed_sketch=504)
    codec = o.turboquant_codec(d, bits, mode, rot_seed=503, sketch_seed=504)
    ref = o.encode(codec, x.double().numpy())
    rec = up(o.pack(codec, ref))
    s, i = tq.search_topk(cb, q.to(DEV), rec, n, k)
    s, i = s.cpu().numpy(), i.cpu().numpy()
    full = o.score(codec, q.double().numpy(), ref)
    rs, ri = o.topk(full, k)
    for r in range(nq):
        tol = 1e-3 * np.linalg.norm(q[r].numpy()) * ref.nx.astype(np.float64)
        kth = rs[r, -1]
        got_set, ref_set = set(i[r].tolist()), set(ri[r].tolist())
        diff = got_set ^ ref_set
        assert all(abs(full[r, j] - kth) <= 2 * tol[j] for j in diff), f"query {r}: top-k differs beyond near-ties"
        assert np.all(np.diff(s[r]) <= 0) and len(got_set) == k
        assert np.all(np.abs(s[r] - full[r, i[r]]) <= tol[i[r]])


@pytest.mark.parametrize("k", [10, 16])
def test_search_topk_equal_scores_take_smallest_ids(k):
    # every key is the same record, so all scores tie: the top-k must be ids
    # 0 .. k-1 (ties go to the smaller id) across all workgroups and lists
    n, d, nq = 70000, 128, 3
    x = synth.iid_gaussian(1, d, 511)
    q = synth.iid_gaussian(nq, d, 512)
    cb = tq.Codebook(d, tq.TQ_PROD, 2, seed_rotation=503, seed_sketch=504)
    codec = o.turboquant_codec(d, 2, "prod", rot_seed=503, sketch_seed=504)
    one = o.encode(codec, x.double().numpy())
    rep = o.Encoded(np.repeat(one.idx, n, axis=0), np.repeat(one.signs, n, axis=0), np.repeat(one.nx, n),
                    np.repeat(one.nr, n), None, None)
    s, i = tq.search_topk(cb, q.to(DEV), up(o.pack(codec, rep)), n, k)
    s, i = s.cpu().numpy(), i.cpu().numpy()
    for r in range(nq):
        assert i[r].tolist() == list(range(k)), i[r].tolist()
        assert np.all(s[r] == s[r, 0])


# -------------------------------------------- full-size decode layer (8B GQA)
def test_gqa_layer_full_size():
    """One decode layer at its full size: 32 q / 8 kv heads, 32768 tokens."""
    Hq, Hkv, T = 32, 8, 32768
    say("full GQA layer: generate")
    law = synth.KVLaw(Hkv, 128, 205)
    K = synth.kv_cache(1, Hkv, T, 128, 201, law)[0]
    V = synth.kv_cache(1, Hkv, T, 128, 251, law)[0]
    q = synth.kv_queries(1, Hq, Hkv, 128, 202, law)
    kcb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=203, seed_sketch=204)
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=203, layout=tq.TQ_LAYOUT_COL)
    kc = o.turboquant_codec(128, 3, "prod", rot_seed=203, sketch_seed=204)
    vc = o.turboquant_codec(128, 4, "mse", rot_seed=203, layout="col")
    say("full GQA layer: encode parity")
    kb, vb = gpu_records(kcb, K), gpu_records(vcb, V)
    per_k, per_v = kcb.records_bytes(T), vcb.records_bytes(T)
    ke, ve, kp, vp = [], [], [], []
    tot = {"K": 0, "V": 0}
    for h in range(Hkv):
        rk = o.encode(kc, K[h].double().numpy())
        rv = o.encode(vc, V[h].double().numpy())
        sk = check_encoded(kc, rk, o.unpack(kc, kb[h * per_k:(h + 1) * per_k], T))
        sv = check_encoded(vc, rv, o.unpack(vc, vb[h * per_v:(h + 1) * per_v], T))
        tot["K"] += sk["band_code_flips"] + sk["band_sign_flips"]
        tot["V"] += sv["band_code_flips"]
        ke.append(rk)
        ve.append(rv)
        kp.append(o.pack(kc, rk))
        vp.append(o.pack(vc, rv))
    say("band flips", tot)
    say("full GQA layer: decode parity")
    scale = 1 / math.sqrt(128)
    ref = o.decode_attention(kc, vc, q[0].double().numpy(), ke, ve, scale)
    out = tq.decode_attend(kcb, vcb, q.to(DEV), up(np.concatenate(kp)), up(np.concatenate(vp)),
                           T, Hkv, scale).cpu().numpy()[0]
    nvmax = max(float(np.max(e.nx.astype(np.float64))) for e in ve)
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"full layer decode: max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3
