"""Outlier-channel split codecs on the GPU against the CPU oracle (TurboQuant
paper review, "Method": for the KV-cache experiments each channel group,
outlier and regular, is quantized by its own TurboQuant instance; 32 channels
at 3 bits + 96 at 2 bits is the 2.5-bit setting).  The outlier channels of
each KV head are the 32 with the largest RMS over a seeded calibration
sample of the synthetic KV law.  Every call goes through the C ABI."""
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


def outlier_channels(law, heads, o_=32, n=2048, seed=900):
    """Per head the o_ channels of largest RMS over a calibration sample."""
    out = []
    for h in range(heads):
        x = law.sample(h, n, torch.Generator().manual_seed(seed + h), "cpu").double()
        rms = x.pow(2).mean(dim=0).sqrt().numpy()
        out.append(np.argsort(-rms, kind="stable")[:o_])
    return np.stack(out).astype(np.int32)


def codecs(ch, bits=(3, 2), mode="prod", seeds=(211, 212), layout="row"):
    m = tq.TQ_PROD if mode == "prod" else tq.TQ_MSE
    cb = tq.Codebook(128, m, bits[1], seed_rotation=seeds[0], seed_sketch=seeds[1], outlier_channels=ch,
                     outlier_bits=bits[0], layout=tq.TQ_LAYOUT_COL if layout == "col" else tq.TQ_LAYOUT_ROW)
    sc = o.outlier_split_codec(128, ch, bits[0], bits[1], mode, rot_seed=seeds[0], sketch_seed=seeds[1],
                               layout=layout)
    return cb, sc


def take(e, n):
    return o.Encoded(e.idx[:n], None if e.signs is None else e.signs[:n], e.nx[:n],
                     None if e.nr is None else e.nr[:n], None if e.y is None else e.y[:n],
                     None if e.z is None else e.z[:n])


def check_split(sc, ref, got):
    return {"outlier": check_encoded(sc.inst_o, ref.o, got.o), "regular": check_encoded(sc.inst_r, ref.r, got.r)}


@pytest.mark.parametrize("mode,dtype", [("prod", torch.bfloat16), ("prod", torch.float32),
                                        ("mse", torch.bfloat16)])
def test_split_encode(mode, dtype):
    H, T = 2, 1000  # 16 tiles, a ragged last tile
    say(f"split encode {mode} {dtype} H={H} T={T}")
    law = synth.KVLaw(H, 128, 905)
    X = synth.kv_cache(1, H, T, 128, 901, law)[0].to(dtype)
    ch = outlier_channels(law, H)
    cb, sc = codecs(ch, bits=(3, 2) if mode == "prod" else (2, 1), mode=mode)
    buf = tq.encode(cb, X.to(DEV)).cpu().numpy()
    per = cb.records_bytes(T)
    assert per == ((T + 63) // 64) * o.split_tile_bytes(sc)
    for h in range(H):
        ref = o.split_encode(sc, X[h].double().numpy(), head=h)
        got = o.split_unpack(sc, buf[h * per:(h + 1) * per], T)
        say(h, check_split(sc, ref, got))
        # the slots past T are zero: repacking what was read gives the same bytes
        assert np.array_equal(o.split_pack(sc, got), buf[h * per:(h + 1) * per])


def test_split_encode_zero_groups():
    # a vector zero on one group: that group encodes y = 0 and stores n_x = 0
    ch = np.arange(0, 128, 4, dtype=np.int32)[None]
    cb, sc = codecs(ch)
    x = torch.randn(70, 128, generator=torch.Generator().manual_seed(3))
    x[3, ch[0]] = 0.0
    reg = np.setdiff1d(np.arange(128), ch[0])
    x[5, reg] = 0.0
    x[7] = 0.0
    got = o.split_unpack(sc, tq.encode(cb, x.to(DEV)).cpu().numpy(), 70)
    assert float(got.o.nx[3]) == 0 and float(got.r.nx[5]) == 0
    assert float(got.o.nx[7]) == 0 and float(got.r.nx[7]) == 0
    s = tq.score(cb, torch.ones(1, 128, device=DEV), up(o.split_pack(sc, got)), 70).cpu().numpy()
    assert s[0, 7] == 0.0


@pytest.mark.parametrize("o_,bits,mode,dtype", [(32, (4, 3), "prod", torch.bfloat16),
                                                 (64, (3, 2), "prod", torch.float32),
                                                 (96, (2, 3), "prod", torch.bfloat16),
                                                 (32, (6, 2), "prod", torch.bfloat16),
                                                 (64, (3, 2), "mse", torch.bfloat16),
                                                 (96, (4, 1), "mse", torch.float32)])
def test_split_encode_general(o_, bits, mode, dtype):
    # outlier counts and bit widths off the 2.5-bit path (up to 5 index bits,
    # bit strings over several 16-byte chunks, a short last chunk)
    H, T = 2, 700
    say(f"general split encode o={o_} bits={bits} {mode} {dtype}")
    law = synth.KVLaw(H, 128, 925)
    X = synth.kv_cache(1, H, T, 128, 921, law)[0].to(dtype)
    ch = outlier_channels(law, H, o_=o_)
    cb, sc = codecs(ch, bits=bits, mode=mode)
    buf = tq.encode(cb, X.to(DEV)).cpu().numpy()
    per = cb.records_bytes(T)
    for h in range(H):
        ref = o.split_encode(sc, X[h].double().numpy(), head=h)
        got = o.split_unpack(sc, buf[h * per:(h + 1) * per], T)
        say(h, check_split(sc, ref, got))
        assert np.array_equal(o.split_pack(sc, got), buf[h * per:(h + 1) * per])


@pytest.mark.parametrize("bits", [(3, 2), (4, 3), (2, 3)])
def test_split_score(bits):
    H, n, nq = 2, 777, 5
    law = synth.KVLaw(H, 128, 915)
    X = synth.kv_cache(1, H, n, 128, 911, law)[0].float()
    q = synth.kv_queries(1, nq, 1, 128, 912, law)[0].float()
    ch = outlier_channels(law, H)
    cb, sc = codecs(ch, bits=bits)
    for h in range(H):
        ref = o.split_encode(sc, X[h].double().numpy(), head=h)
        s = tq.score(cb, q.to(DEV), up(o.split_pack(sc, ref)), n, head=h).cpu().numpy()
        want = o.split_score(sc, q.double().numpy(), ref, head=h)
        nx = np.sqrt(ref.o.nx.astype(np.float64) ** 2 + ref.r.nx.astype(np.float64) ** 2)
        say(bits, h, "max scaled error", check_scores(s, want, q.numpy(), nx))


def test_split_topk():
    n, nq, k = 5000, 6, 10
    law = synth.KVLaw(1, 128, 925)
    X = synth.kv_cache(1, 1, n, 128, 921, law)[0, 0].float()
    q = synth.kv_queries(1, nq, 1, 128, 922, law)[0].float()
    cb, sc = codecs(outlier_channels(law, 1))
    ref = o.split_encode(sc, X.double().numpy())
    s, i = tq.search_topk(cb, q.to(DEV), up(o.split_pack(sc, ref)), n, k)
    s, i = s.cpu().numpy(), i.cpu().numpy()
    full = o.split_score(sc, q.double().numpy(), ref)
    rs, ri = o.topk(full, k)
    # a candidate's score tolerance is 1e-3 ||q|| times its own norm (both
    # instances' n_x, which bound its reconstruction's length)
    nxv = ref.o.nx.astype(np.float64) + ref.r.nx.astype(np.float64)
    for r in range(nq):
        tol = 1e-3 * np.linalg.norm(q[r].numpy()) * nxv
        near = np.abs(full[r] - rs[r, -1]) <= 2 * tol
        diff = set(i[r].tolist()) ^ set(ri[r].tolist())
        assert all(near[j] for j in diff), [(j, full[r, j] - rs[r, -1], tol[j]) for j in diff]
        assert np.all(np.diff(s[r]) <= 0)
        assert len(set(i[r].tolist())) == k
        assert np.all(np.abs(s[r] - full[r, i[r]]) <= tol[i[r]])


def _decode(B, Hq, Hkv, T, seq_lens, kbits=(3, 2)):
    law = synth.KVLaw(Hkv, 128, 935)
    K = synth.kv_cache(B, Hkv, T, 128, 931, law)
    V = synth.kv_cache(B, Hkv, T, 128, 932, law)
    q = synth.kv_queries(B, Hq, Hkv, 128, 933, law)
    kcb, sc = codecs(outlier_channels(law, Hkv), bits=kbits)
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=937, layout=tq.TQ_LAYOUT_COL)
    vc = o.turboquant_codec(128, 4, "mse", rot_seed=937, layout="col")
    ke = [[o.split_encode(sc, K[b, g].double().numpy(), head=g) for g in range(Hkv)] for b in range(B)]
    ve = [[o.encode(vc, V[b, g].double().numpy()) for g in range(Hkv)] for b in range(B)]
    kbuf = np.concatenate([o.split_pack(sc, e) for row in ke for e in row])
    vbuf = np.concatenate([o.pack(vc, e) for row in ve for e in row])
    scale = 1 / math.sqrt(128)
    ref = np.zeros((B, Hq, 128))
    for b in range(B):
        L_ = seq_lens[b]
        if L_ == 0:
            continue
        kk = [o.SplitEncoded(take(e.o, L_), take(e.r, L_)) for e in ke[b]]
        vv = [take(e, L_) for e in ve[b]]
        ref[b] = o.split_decode_attention(sc, vc, q[b].double().numpy(), kk, vv, scale)
    out = tq.decode_attend(kcb, vcb, q.to(DEV), up(kbuf), up(vbuf), T, Hkv, scale,
                           seq_lens=torch.tensor(seq_lens, dtype=torch.int32, device=DEV)).cpu().numpy()
    nvmax = max(float(np.max(e.nx.astype(np.float64))) for row in ve for e in row)
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"split decode B={B} Hq={Hq} Hkv={Hkv} T={T} bits={kbits}: max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3


def test_split_decode_gqa():
    _decode(2, 8, 2, 700, [700, 129])


def test_split_decode_other_bits():
    # 3 index bits on the outlier channels: the general decode kernel
    _decode(1, 4, 1, 300, [300], kbits=(4, 3))


@pytest.mark.parametrize("B,Hq,Hkv,T,lens", [(1, 2, 1, 300, [300]), (2, 4, 4, 1500, [1500, 777]),
                                             (3, 16, 4, 200, [200, 1, 65])])
def test_split_decode_mfma_shapes(B, Hq, Hkv, T, lens):
    # 2.5-bit keys on the MFMA decode: group sizes 2, 1, 4; one split per
    # sequence (fused epilogue) and several
    _decode(B, Hq, Hkv, T, lens)


@pytest.mark.parametrize("bits", [(3, 2), (4, 3)])
def test_split_append(bits):
    B, H, cap, steps = 3, 2, 200, 5
    L0 = [0, 62, 128]
    law = synth.KVLaw(H, 128, 945)
    X = synth.kv_cache(B, H, cap, 128, 941, law)
    cb, sc = codecs(outlier_channels(law, H), bits=bits)
    full = {(b, h): o.split_encode(sc, X[b, h].double().numpy(), head=h) for b in range(B) for h in range(H)}
    per = cb.records_bytes(cap)
    rec = np.zeros(B * H * per, np.uint8)
    for b in range(B):
        for h in range(H):
            if L0[b]:
                p = o.split_pack(sc, o.SplitEncoded(take(full[b, h].o, L0[b]), take(full[b, h].r, L0[b])))
                rec[(b * H + h) * per:(b * H + h) * per + len(p)] = p
    rec = up(rec)
    for s in range(steps):
        pos = torch.tensor([L0[b] + s for b in range(B)], dtype=torch.int32, device=DEV)
        tq.append(cb, torch.stack([X[b, :, L0[b] + s] for b in range(B)]).to(DEV), rec, pos, cap)
    got_all = rec.cpu().numpy()
    for b in range(B):
        for h in range(H):
            n = L0[b] + steps
            buf = got_all[(b * H + h) * per:(b * H + h + 1) * per]
            got = o.split_unpack(sc, buf, n)
            ref = o.SplitEncoded(take(full[b, h].o, n), take(full[b, h].r, n))
            say(bits, b, h, check_split(sc, ref, got))
            want = np.zeros(per, np.uint8)
            p = o.split_pack(sc, got)
            want[:len(p)] = p
            assert np.array_equal(buf, want)


def test_gqa_outlier_full_size():
    """The 2.5-bit split layer at its full size (32 q / 8 kv heads, 32768
    tokens): every key's records against the oracle, then the decode step."""
    Hq, Hkv, T = 32, 8, 32768
    say("split full layer: generate")
    law = synth.KVLaw(Hkv, 128, 205)
    K = synth.kv_cache(1, Hkv, T, 128, 201, law)[0]
    V = synth.kv_cache(1, Hkv, T, 128, 251, law)[0]
    q = synth.kv_queries(1, Hq, Hkv, 128, 202, law)
    kcb, sc = codecs(outlier_channels(law, Hkv), seeds=(203, 204))
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=203, layout=tq.TQ_LAYOUT_COL)
    vc = o.turboquant_codec(128, 4, "mse", rot_seed=203, layout="col")
    say("split full layer: encode parity")
    kb = tq.encode(kcb, K.to(DEV)).cpu().numpy()
    per = kcb.records_bytes(T)
    ke, ve, tot = [], [], 0
    for h in range(Hkv):
        ref = o.split_encode(sc, K[h].double().numpy(), head=h)
        st = check_split(sc, ref, o.split_unpack(sc, kb[h * per:(h + 1) * per], T))
        tot += sum(v["band_code_flips"] + v["band_sign_flips"] for v in st.values())
        ke.append(ref)
        ve.append(o.encode(vc, V[h].double().numpy()))
    say("band flips", tot)
    say("split full layer: decode parity")
    scale = 1 / math.sqrt(128)
    ref = o.split_decode_attention(sc, vc, q[0].double().numpy(), ke, ve, scale)
    out = tq.decode_attend(kcb, vcb, q.to(DEV), torch.from_numpy(kb).to(DEV),
                           up(np.concatenate([o.pack(vc, e) for e in ve])), T, Hkv, scale).cpu().numpy()[0]
    nvmax = max(float(np.max(e.nx.astype(np.float64))) for e in ve)
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"split full layer decode: max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3


def _decode_split_values(B, Hq, Hkv, T, seq_lens, kbits=(3, 2), vbits=(3, 2), split_keys=True, vlayout="row"):
    """Decode over values of an outlier-split mse codec (ROW records; the
    paper review's KV-cache setting splits the values' channels too)."""
    law = synth.KVLaw(Hkv, 128, 955)
    K = synth.kv_cache(B, Hkv, T, 128, 951, law)
    V = synth.kv_cache(B, Hkv, T, 128, 952, law)
    q = synth.kv_queries(B, Hq, Hkv, 128, 953, law)
    ch = outlier_channels(law, Hkv, seed=960)
    if split_keys:
        kcb, kc = codecs(ch, bits=kbits)
        kenc = lambda x, g: o.split_encode(kc, x, head=g)
        kpack = lambda e: o.split_pack(kc, e)
        ktake = lambda e, n: o.SplitEncoded(take(e.o, n), take(e.r, n))
    else:
        kcb = tq.Codebook(128, tq.TQ_PROD, kbits[0], seed_rotation=211, seed_sketch=212)
        kc = o.turboquant_codec(128, kbits[0], "prod", rot_seed=211, sketch_seed=212)
        kenc = lambda x, g: o.encode(kc, x)
        kpack = lambda e: o.pack(kc, e)
        ktake = take
    vcb, vc = codecs(ch, bits=vbits, mode="mse", seeds=(957, 958), layout=vlayout)
    ke = [[kenc(K[b, g].double().numpy(), g) for g in range(Hkv)] for b in range(B)]
    ve = [[o.split_encode(vc, V[b, g].double().numpy(), head=g) for g in range(Hkv)] for b in range(B)]
    kbuf = np.concatenate([kpack(e) for row in ke for e in row])
    vbuf = np.concatenate([o.split_pack(vc, e) for row in ve for e in row])
    # the value records as the GPU encodes them match the oracle's
    gv = tq.encode(vcb, V.to(DEV)).cpu().numpy()
    per = vcb.records_bytes(T)
    for b in range(B):
        for g in range(Hkv):
            got = o.split_unpack(vc, gv[(b * Hkv + g) * per:(b * Hkv + g + 1) * per], T)
            check_split(vc, ve[b][g], got)
    scale = 1 / math.sqrt(128)
    ref = np.zeros((B, Hq, 128))
    for b in range(B):
        L_ = seq_lens[b]
        if L_ == 0:
            continue
        kk = [ktake(e, L_) for e in ke[b]]
        vv = [o.SplitEncoded(take(e.o, L_), take(e.r, L_)) for e in ve[b]]
        ref[b] = o.split_decode_attention(kc, vc, q[b].double().numpy(), kk, vv, scale)
    out = tq.decode_attend(kcb, vcb, q.to(DEV), up(kbuf), up(vbuf), T, Hkv, scale,
                           seq_lens=torch.tensor(seq_lens, dtype=torch.int32, device=DEV)).cpu().numpy()
    nvmax = max(max(float(np.max(e.o.nx.astype(np.float64))), float(np.max(e.r.nx.astype(np.float64))))
                for row in ve for e in row)
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"split-value decode B={B} Hq={Hq} Hkv={Hkv} T={T} k={kbits} v={vbits} {vlayout} split keys={split_keys}: "
        f"max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3
    if any(L_ == 0 for L_ in seq_lens):
        assert not np.any(out[[b for b in range(B) if seq_lens[b] == 0]])


@pytest.mark.parametrize("B,Hq,Hkv,T,lens,kbits,vbits,sk", [
    (2, 8, 2, 700, [700, 129], (3, 2), (3, 2), True),   # 2.5-bit K and V
    (3, 4, 4, 300, [300, 0, 65], (3, 2), (4, 3), True),  # 3.5-bit values, an empty sequence
    (1, 2, 1, 1000, [1000], (3, 3), (2, 1), False),      # plain prod keys, 1.5-bit values
])
def test_split_value_decode(B, Hq, Hkv, T, lens, kbits, vbits, sk):
    _decode_split_values(B, Hq, Hkv, T, lens, kbits, vbits, sk)


def test_row_value_decode():
    # values in ROW records of a uniform mse codec (any index bits) on the
    # general decode kernel
    B, Hq, Hkv, T = 2, 8, 2, 500
    lens = [500, 333]
    law = synth.KVLaw(Hkv, 128, 965)
    K = synth.kv_cache(B, Hkv, T, 128, 961, law)
    V = synth.kv_cache(B, Hkv, T, 128, 962, law)
    q = synth.kv_queries(B, Hq, Hkv, 128, 963, law)
    kcb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=966, seed_sketch=967)
    kc = o.turboquant_codec(128, 3, "prod", rot_seed=966, sketch_seed=967)
    for vb in (3, 4):
        say(f"row-value decode b={vb}")
        vcb = tq.Codebook(128, tq.TQ_MSE, vb, seed_rotation=968)
        vc = o.turboquant_codec(128, vb, "mse", rot_seed=968)
        kb = tq.encode(kcb, K.to(DEV))
        vbuf = tq.encode(vcb, V.to(DEV))
        kper, vper = kcb.records_bytes(T), vcb.records_bytes(T)
        kcpu, vcpu = kb.cpu().numpy(), vbuf.cpu().numpy()
        scale = 1 / math.sqrt(128)
        out = tq.decode_attend(kcb, vcb, q.to(DEV), kb, vbuf, T, Hkv, scale,
                               seq_lens=torch.tensor(lens, dtype=torch.int32, device=DEV)).cpu().numpy()
        nvmax, err = 0.0, 0.0
        for b in range(B):
            ke = [o.unpack(kc, kcpu[(b * Hkv + g) * kper:(b * Hkv + g + 1) * kper], lens[b]) for g in range(Hkv)]
            ve = [o.unpack(vc, vcpu[(b * Hkv + g) * vper:(b * Hkv + g + 1) * vper], lens[b]) for g in range(Hkv)]
            for g in range(Hkv):
                check_encoded(vc, o.encode(vc, V[b, g, :lens[b]].double().numpy()), ve[g])
            ref = o.decode_attention(kc, vc, q[b].double().numpy(), ke, ve, scale)
            nvmax = max(nvmax, max(float(np.max(e.nx.astype(np.float64))) for e in ve))
            err = max(err, float(np.max(np.abs(out[b] - ref))))
        say(f"row-value decode b={vb}: max |out - ref| / max n_v = {err / nvmax:.3g}")
        assert err / nvmax <= 1e-3


@pytest.mark.parametrize("vlayout", ["row", "col"])
def test_gqa_outlier_kv_full_size(vlayout):
    """2.5-bit keys and values (both split: 32 outlier channels at 3 bits, 96
    at 2) on the full layer, 32 q / 8 kv heads, 32768 tokens: the GPU value
    records (row records: general decode kernel; col: MFMA decode) against
    the oracle, then the decode step."""
    Hq, Hkv, T = 32, 8, 32768
    say("split K+V full layer: generate")
    law = synth.KVLaw(Hkv, 128, 205)
    K = synth.kv_cache(1, Hkv, T, 128, 201, law)[0]
    V = synth.kv_cache(1, Hkv, T, 128, 251, law)[0]
    q = synth.kv_queries(1, Hq, Hkv, 128, 202, law)
    ch = outlier_channels(law, Hkv)
    kcb, kc = codecs(ch, seeds=(203, 204))
    vcb, vc = codecs(ch, mode="mse", seeds=(213, 214), layout=vlayout)
    say("split K+V full layer: encode")
    kb, vb = tq.encode_kv(kcb, vcb, K.to(torch.bfloat16).to(DEV), V.to(torch.bfloat16).to(DEV))
    kb, vb = kb.cpu().numpy(), vb.cpu().numpy()
    kper, vper = kcb.records_bytes(T), vcb.records_bytes(T)
    ke, ve, tot = [], [], 0
    for h in range(Hkv):
        xk = K[h].to(torch.bfloat16).double().numpy()
        xv = V[h].to(torch.bfloat16).double().numpy()
        rk, rv = o.split_encode(kc, xk, head=h), o.split_encode(vc, xv, head=h)
        st = check_split(vc, rv, o.split_unpack(vc, vb[h * vper:(h + 1) * vper], T))
        tot += sum(v["band_code_flips"] for v in st.values())
        ke.append(o.split_unpack(kc, kb[h * kper:(h + 1) * kper], T))
        ve.append(o.split_unpack(vc, vb[h * vper:(h + 1) * vper], T))
    say("value band flips", tot)
    say("split K+V full layer: decode parity")
    scale = 1 / math.sqrt(128)
    ref = o.split_decode_attention(kc, vc, q[0].double().numpy(), ke, ve, scale)
    out = tq.decode_attend(kcb, vcb, q.to(DEV), torch.from_numpy(kb).to(DEV), torch.from_numpy(vb).to(DEV),
                           T, Hkv, scale).cpu().numpy()[0]
    nvmax = max(max(float(np.max(e.o.nx.astype(np.float64))), float(np.max(e.r.nx.astype(np.float64))))
                for e in ve)
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"split K+V full layer ({vlayout} values) decode: max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3


@pytest.mark.parametrize("vlayout", ["row", "col"])
def test_split_kv_decode_step(vlayout):
    # append-on-decode with split keys and split values: each step writes the
    # new key and value into slot seq_lens[b] (split ROW records, tq_append)
    # and attends over seq_lens[b] + 1 tokens
    B, H, Hq, cap, steps = 2, 2, 8, 200, 3
    L0 = [0, 130]
    law = synth.KVLaw(H, 128, 975)
    K = synth.kv_cache(B, H, cap, 128, 971, law)
    V = synth.kv_cache(B, H, cap, 128, 972, law)
    ch = outlier_channels(law, H, seed=980)
    kcb, kc = codecs(ch, seeds=(973, 974))
    vcb, vc = codecs(ch, mode="mse", seeds=(976, 977), layout=vlayout)
    kf = {(b, h): o.split_encode(kc, K[b, h].double().numpy(), head=h) for b in range(B) for h in range(H)}
    vf = {(b, h): o.split_encode(vc, V[b, h].double().numpy(), head=h) for b in range(B) for h in range(H)}
    kper, vper = kcb.records_bytes(cap), vcb.records_bytes(cap)
    kr, vr = np.zeros(B * H * kper, np.uint8), np.zeros(B * H * vper, np.uint8)
    for b in range(B):
        for h in range(H):
            if L0[b]:
                p = o.split_pack(kc, o.SplitEncoded(take(kf[b, h].o, L0[b]), take(kf[b, h].r, L0[b])))
                kr[(b * H + h) * kper:(b * H + h) * kper + len(p)] = p
                p = o.split_pack(vc, o.SplitEncoded(take(vf[b, h].o, L0[b]), take(vf[b, h].r, L0[b])))
                vr[(b * H + h) * vper:(b * H + h) * vper + len(p)] = p
    kr, vr = up(kr), up(vr)
    scale = 1 / math.sqrt(128)
    for s_ in range(steps):
        lens = [L0[b] + s_ for b in range(B)]
        q = synth.kv_queries(B, Hq, H, 128, 985 + s_, law)
        kn = torch.stack([K[b, :, lens[b]] for b in range(B)]).to(DEV)
        vn = torch.stack([V[b, :, lens[b]] for b in range(B)]).to(DEV)
        out = tq.decode_step(kcb, vcb, q.to(DEV), kn, vn, kr, vr, cap, H, scale,
                             torch.tensor(lens, dtype=torch.int32, device=DEV)).cpu().numpy()
        nvmax, err = 0.0, 0.0
        for b in range(B):
            n = lens[b] + 1
            kk = [o.SplitEncoded(take(kf[b, h].o, n), take(kf[b, h].r, n)) for h in range(H)]
            vv = [o.SplitEncoded(take(vf[b, h].o, n), take(vf[b, h].r, n)) for h in range(H)]
            ref = o.split_decode_attention(kc, vc, q[b].double().numpy(), kk, vv, scale)
            err = max(err, float(np.max(np.abs(out[b] - ref))))
            nvmax = max(nvmax, max(max(float(np.max(e.o.nx.astype(np.float64))),
                                       float(np.max(e.r.nx.astype(np.float64)))) for e in vv))
        say(f"split K+V ({vlayout} values) decode step {s_}: max |out - ref| / max n_v = {err / nvmax:.3g}")
        assert err / nvmax <= 1e-3
    # the value records now hold L0 + steps tokens each, as the oracle encodes them
    vall = vr.cpu().numpy()
    for b in range(B):
        for h in range(H):
            n = L0[b] + steps
            got = o.split_unpack(vc, vall[(b * H + h) * vper:(b * H + h + 1) * vper], n)
            check_split(vc, o.SplitEncoded(take(vf[b, h].o, n), take(vf[b, h].r, n)), got)


@pytest.mark.parametrize("B,Hq,Hkv,T,lens,kbits,sk", [
    (2, 8, 2, 700, [700, 129], (3, 2), True),     # split keys, several splits per sequence
    (3, 4, 4, 300, [300, 0, 65], (3, 2), True),   # an empty sequence, group size 1
    (1, 2, 1, 1000, [1000], (3, 3), False),       # 2-bit TurboQuant-prod keys, group size 2
    (66, 4, 4, 129, [129] * 66, (3, 2), True),    # one split per sequence (4-wave form)
    (1, 4, 1, 2500, [2500], (3, 2), True),        # 8-wave workgroups over 16-tile splits
])
def test_split_col_value_decode(B, Hq, Hkv, T, lens, kbits, sk):
    # 2.5-bit split values in col records: the GPU encode of the records
    # against the oracle, then the MFMA decode
    _decode_split_values(B, Hq, Hkv, T, lens, kbits, (3, 2), sk, vlayout="col")
