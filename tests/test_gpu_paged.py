"""Paged KV caches and the decode step with append-on-decode on the GPU,
against the CPU oracle (TurboQuant paper review, "Comparison": tokens
generated during decoding are quantized too).  Records are packed by the
oracle into pages of a pool in a seeded random order; the block table maps
each (sequence, KV head) to its pages."""
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
D = 128


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def take(e, n):
    return o.Encoded(e.idx[:n], None if e.signs is None else e.signs[:n], e.nx[:n],
                     None if e.nr is None else e.nr[:n], None if e.y is None else e.y[:n],
                     None if e.z is None else e.z[:n])


def codecs(kind):
    if kind == "prod3":
        kcb = tq.Codebook(D, tq.TQ_PROD, 3, seed_rotation=603, seed_sketch=604)
        kc = o.turboquant_codec(D, 3, "prod", rot_seed=603, sketch_seed=604)
        pack, enc = o.pack, (lambda x, h: o.encode(kc, x))
    else:  # split keys with 3 outlier index bits: the general decode kernel
        ch = np.arange(0, D, 4, dtype=np.int32)
        kcb = tq.Codebook(D, tq.TQ_PROD, 3, seed_rotation=603, seed_sketch=604, outlier_channels=ch,
                          outlier_bits=4)
        kc = o.outlier_split_codec(D, ch, 4, 3, "prod", rot_seed=603, sketch_seed=604)
        pack, enc = o.split_pack, (lambda x, h: o.split_encode(kc, x))
    vcb = tq.Codebook(D, tq.TQ_MSE, 4, seed_rotation=607, layout=tq.TQ_LAYOUT_COL)
    vc = o.turboquant_codec(D, 4, "mse", rot_seed=607, layout="col")
    return kcb, kc, pack, enc, vcb, vc


def paged(records_per_set, tile_bytes, page_tiles, rng, spare=5):
    """Pool bytes and block table [sets][max_pages] for per-set record buffers
    (each a whole number of tiles), pages placed in a random order."""
    sets = len(records_per_set)
    ntiles = len(records_per_set[0]) // tile_bytes
    max_pages = (ntiles + page_tiles - 1) // page_tiles
    npages = sets * max_pages + spare
    order = rng.permutation(npages)
    page_bytes = page_tiles * tile_bytes
    pool = np.zeros(npages * page_bytes, np.uint8)
    table = np.zeros((sets, max_pages), np.int32)
    k = 0
    for s_, rec in enumerate(records_per_set):
        for p in range(max_pages):
            pg = int(order[k])
            k += 1
            table[s_, p] = pg
            chunk = rec[p * page_bytes:(p + 1) * page_bytes]
            pool[pg * page_bytes:pg * page_bytes + len(chunk)] = chunk
    return pool, table


def set_records(pack_fn, codec, enc, cb, cap):
    buf = np.zeros(cb.records_bytes(cap), np.uint8)
    if enc is not None:
        p = pack_fn(codec, enc)
        buf[:len(p)] = p
    return buf


def reference(kc, vc, q, kfull, vfull, lens, B, H, split):
    scale = 1 / math.sqrt(D)
    out = np.zeros((B, q.shape[1], D))
    for b in range(B):
        if lens[b] == 0:
            continue
        if split:
            kk = [o.SplitEncoded(take(kfull[b, h].o, lens[b]), take(kfull[b, h].r, lens[b])) for h in range(H)]
            out[b] = o.split_decode_attention(kc, vc, q[b].double().numpy(), kk,
                                              [take(vfull[b, h], lens[b]) for h in range(H)], scale)
        else:
            out[b] = o.decode_attention(kc, vc, q[b].double().numpy(), [take(kfull[b, h], lens[b]) for h in range(H)],
                                        [take(vfull[b, h], lens[b]) for h in range(H)], scale)
    return out


@pytest.mark.parametrize("kind,page_tiles", [("prod3", 1), ("prod3", 4), ("split43", 2)])
def test_paged_decode(kind, page_tiles):
    B, H, Hq, cap = 3, 2, 8, 1000
    lens = [1000, 1, 577]
    rng = np.random.default_rng(page_tiles)
    law = synth.KVLaw(H, D, 615)
    K = synth.kv_cache(B, H, cap, D, 611, law)
    V = synth.kv_cache(B, H, cap, D, 612, law)
    q = synth.kv_queries(B, Hq, H, D, 613, law)
    kcb, kc, pack, enc, vcb, vc = codecs(kind)
    kfull = {(b, h): enc(K[b, h].double().numpy(), h) for b in range(B) for h in range(H)}
    vfull = {(b, h): o.encode(vc, V[b, h].double().numpy()) for b in range(B) for h in range(H)}
    krec = [set_records(pack, kc, kfull[b, h], kcb, cap) for b in range(B) for h in range(H)]
    vrec = [set_records(o.pack, vc, vfull[b, h], vcb, cap) for b in range(B) for h in range(H)]
    kpool, table = paged(krec, kcb.tile_bytes, page_tiles, rng)
    vpool, vtable = paged(vrec, vcb.tile_bytes, page_tiles, np.random.default_rng(page_tiles))
    assert np.array_equal(table, vtable)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(D)
    out = tq.decode_attend(kcb, vcb, q.to(DEV), torch.from_numpy(kpool).to(DEV), torch.from_numpy(vpool).to(DEV),
                           cap, H, scale, seq_lens=sl, block_table=torch.from_numpy(table).to(DEV),
                           page_tiles=page_tiles).cpu().numpy()
    flat = tq.decode_attend(kcb, vcb, q.to(DEV), torch.from_numpy(np.concatenate(krec)).to(DEV),
                            torch.from_numpy(np.concatenate(vrec)).to(DEV), cap, H, scale, seq_lens=sl).cpu().numpy()
    ref = reference(kc, vc, q, kfull, vfull, lens, B, H, kind != "prod3")
    nvmax = max(float(np.max(e.nx.astype(np.float64))) for e in vfull.values())
    err = np.max(np.abs(out - ref)) / nvmax
    say(f"paged decode {kind} page_tiles={page_tiles}: max |out - ref| / max n_v = {err:.3g}")
    assert err <= 1e-3
    assert np.array_equal(out, flat)  # the same tiles in the same order


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_decode_step(layout):
    B, H, Hq, cap, steps = 3, 2, 8, 300, 3
    L0 = [0, 63, 200]
    page_tiles = 2
    rng = np.random.default_rng(5)
    law = synth.KVLaw(H, D, 625)
    K = synth.kv_cache(B, H, cap, D, 621, law)
    V = synth.kv_cache(B, H, cap, D, 622, law)
    kcb, kc, pack, enc, vcb, vc = codecs("prod3")
    kfull = {(b, h): o.encode(kc, K[b, h].double().numpy()) for b in range(B) for h in range(H)}
    vfull = {(b, h): o.encode(vc, V[b, h].double().numpy()) for b in range(B) for h in range(H)}
    krec = [set_records(o.pack, kc, take(kfull[b, h], L0[b]) if L0[b] else None, kcb, cap)
            for b in range(B) for h in range(H)]
    vrec = [set_records(o.pack, vc, take(vfull[b, h], L0[b]) if L0[b] else None, vcb, cap)
            for b in range(B) for h in range(H)]
    kw = dict()
    if layout == "paged":
        kpool, table = paged(krec, kcb.tile_bytes, page_tiles, rng)
        vpool, _ = paged(vrec, vcb.tile_bytes, page_tiles, np.random.default_rng(5))
        kr, vr = torch.from_numpy(kpool).to(DEV), torch.from_numpy(vpool).to(DEV)
        kw = dict(block_table=torch.from_numpy(table).to(DEV), page_tiles=page_tiles)
    else:
        kr = torch.from_numpy(np.concatenate(krec)).to(DEV)
        vr = torch.from_numpy(np.concatenate(vrec)).to(DEV)
    scale = 1 / math.sqrt(D)
    for s_ in range(steps):
        lens = [L0[b] + s_ for b in range(B)]
        q = synth.kv_queries(B, Hq, H, D, 630 + s_, law)
        kn = torch.stack([K[b, :, lens[b]] for b in range(B)]).to(DEV)
        vn = torch.stack([V[b, :, lens[b]] for b in range(B)]).to(DEV)
        out = tq.decode_step(kcb, vcb, q.to(DEV), kn, vn, kr, vr, cap, H, scale,
                             torch.tensor(lens, dtype=torch.int32, device=DEV), **kw).cpu().numpy()
        ref = reference(kc, vc, q, kfull, vfull, [n + 1 for n in lens], B, H, False)
        nvmax = max(float(np.max(e.nx.astype(np.float64))) for e in vfull.values())
        err = np.max(np.abs(out - ref)) / nvmax
        say(f"decode step {layout} {s_}: max |out - ref| / max n_v = {err:.3g}")
        assert err <= 1e-3
    # the records now hold L0 + steps tokens each, as the oracle encodes them
    kall, vall = kr.cpu().numpy(), vr.cpu().numpy()
    for b in range(B):
        for h in range(H):
            n = L0[b] + steps
            s_ = b * H + h
            if layout == "paged":
                kb = np.concatenate([kall[pg * page_tiles * kcb.tile_bytes:(pg + 1) * page_tiles * kcb.tile_bytes]
                                     for pg in table[s_]])
                vb = np.concatenate([vall[pg * page_tiles * vcb.tile_bytes:(pg + 1) * page_tiles * vcb.tile_bytes]
                                     for pg in table[s_]])
            else:
                kb = kall[s_ * kcb.records_bytes(cap):(s_ + 1) * kcb.records_bytes(cap)]
                vb = vall[s_ * vcb.records_bytes(cap):(s_ + 1) * vcb.records_bytes(cap)]
            check_encoded(kc, take(kfull[b, h], n), o.unpack(kc, kb, n))
            check_encoded(vc, take(vfull[b, h], n), o.unpack(vc, vb, n))


def test_paging_argument_errors():
    kcb, kc, pack, enc, vcb, vc = codecs("prod3")
    q = torch.zeros(1, 4, D, device=DEV)
    rec = torch.zeros(kcb.records_bytes(128) * 4, dtype=torch.uint8, device=DEV)
    vrec = torch.zeros(vcb.records_bytes(128) * 4, dtype=torch.uint8, device=DEV)
    bt = torch.zeros(1, 2, dtype=torch.int32, device=DEV)
    with pytest.raises(tq.TQError):  # pages of 3 tiles: not a power of two
        tq.decode_attend(kcb, vcb, q, rec, vrec, 128, 1, 0.1, block_table=bt, page_tiles=3)
    with pytest.raises(tq.TQError):  # 1 page of 1 tile cannot hold 128 tokens
        tq.decode_attend(kcb, vcb, q, rec, vrec, 128, 1, 0.1, block_table=bt[:, :1], page_tiles=1)
