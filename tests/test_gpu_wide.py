"""Parity of the wide-vector path (d = 1536, the vector-search width) against
the oracle on MI355X: encode, scoring and top-k across the row chunks the
library processes at a time."""
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
D = 1536


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def up(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def tiles(codec, buf, t0, t1):
    tb = o.tile_bytes(codec)
    return buf[t0 * tb:t1 * tb]


def encoded_rows(enc, rows):
    return o.Encoded(enc.idx[rows], None if enc.signs is None else enc.signs[rows], enc.nx[rows],
                     None if enc.nr is None else enc.nr[rows], enc.y[rows],
                     None if enc.z is None else enc.z[rows])


def test_encode_d1536_special_rows():
    """Rows of zeros, of -0, one nonzero coordinate, and magnitudes near 1e-30
    and 1e3 (70 rows, fp32), against the oracle; zero rows store n_x = 0."""
    g = torch.Generator().manual_seed(43)
    x = torch.randn(70, D, generator=g)
    x[2] = 0.0
    x[3] = -torch.zeros(D)
    x[4] = 0.0
    x[4, 700] = 3.0
    x[5] *= 1e-30
    x[6] *= 1e3
    cb = tq.Codebook(D, tq.TQ_PROD, 2, seed_rotation=503, seed_sketch=504)
    codec = o.turboquant_codec(D, 2, "prod", rot_seed=503, sketch_seed=504)
    rec = tq.encode(cb, x.to(DEV))
    torch.cuda.synchronize()
    ref = o.encode(codec, x.double().numpy())
    got = o.unpack(codec, rec.cpu().numpy(), 70)
    say(check_encoded(codec, ref, got))
    assert float(got.nx[2]) == 0.0 and float(got.nx[3]) == 0.0


@pytest.mark.parametrize("bits", [2, 4])
def test_encode_d1536(bits):
    """1000 vectors: 16 tiles with a ragged tail, against the oracle."""
    say(f"wide encode prod b={bits} n=1000")
    law = synth.LowRankLaw(D, 64, synth.seed(5, "rotation") + 50)
    x = synth.lowrank_vectors(1000, law, synth.seed(5, "data"))
    cb = tq.Codebook(D, tq.TQ_PROD, bits, seed_rotation=503, seed_sketch=504)
    codec = o.turboquant_codec(D, bits, "prod", rot_seed=503, sketch_seed=504)
    rec = tq.encode(cb, x.to(DEV))
    torch.cuda.synchronize()
    buf = rec.cpu().numpy()
    ref = o.encode(codec, x.double().numpy())
    got = o.unpack(codec, buf, 1000)
    say(check_encoded(codec, ref, got))
    assert np.array_equal(o.pack(codec, got), buf)


def test_encode_d1536_chunk_boundary():
    """16484 vectors span two row chunks; the tiles at the start, around the
    chunk edge and at the end are checked against the oracle."""
    n = 16384 + 100
    say(f"wide encode across a chunk edge n={n}")
    law = synth.LowRankLaw(D, 64, 551)
    x = synth.lowrank_vectors(n, law, 552)
    cb = tq.Codebook(D, tq.TQ_PROD, 2, seed_rotation=553, seed_sketch=554)
    codec = o.turboquant_codec(D, 2, "prod", rot_seed=553, sketch_seed=554)
    buf = tq.encode(cb, x.to(DEV)).cpu().numpy()
    assert len(buf) == cb.records_bytes(n)
    for t0, t1 in [(0, 1), (254, 258), ((n - 1) // 64, (n + 63) // 64)]:
        rows = np.arange(t0 * 64, min(n, t1 * 64))
        ref = o.encode(codec, x[rows].double().numpy())
        got = o.unpack(codec, tiles(codec, buf, t0, t1), len(rows))
        say(t0, t1, check_encoded(codec, ref, got))
        if t1 * 64 > n:
            assert np.array_equal(o.pack(codec, got), tiles(codec, buf, t0, t1))


def synthetic_db(codec, n, seed, part=8192):
    """Oracle-packed records of arbitrary stored codes, with their Encoded parts."""
    bufs, encs = [], []
    levels = len(codec.centroids[0][0])
    for i, r0 in enumerate(range(0, n, part)):
        r1 = min(n, r0 + part)
        idx, signs, nx, nr = synth.random_codes(r1 - r0, codec.d, levels, codec.m, seed + i)
        e = o.Encoded(idx, signs, nx, nr, None, None)
        encs.append(e)
        bufs.append(o.pack(codec, e))
    return np.concatenate(bufs), encs


def oracle_scores(codec, q, encs):
    return np.concatenate([o.score(codec, q, e) for e in encs], axis=1)


@pytest.mark.parametrize("bits", [2, 4])
def test_score_d1536(bits):
    """16 queries x 70000 stored codes (two key chunks, ragged tail)."""
    n = 70000
    say(f"wide score b={bits} 16 x {n}")
    cb = tq.Codebook(D, tq.TQ_PROD, bits, seed_rotation=563, seed_sketch=564)
    codec = o.turboquant_codec(D, bits, "prod", rot_seed=563, sketch_seed=564)
    buf, encs = synthetic_db(codec, n, 565)
    law = synth.LowRankLaw(D, 64, 566)
    q = synth.lowrank_vectors(16, law, 567)
    s = tq.score(cb, q.to(DEV), up(buf), n).cpu().numpy()
    ref = oracle_scores(codec, q.double().numpy(), encs)
    nx = np.concatenate([e.nx for e in encs])
    say("max scaled error", check_scores(s, ref, q.numpy(), nx))


def test_topk_d1536():
    """Top-10 of 8 queries over 140000 stored codes (three key chunks)."""
    n, k = 140000, 10
    say(f"wide top-k 8 x {n}")
    cb = tq.Codebook(D, tq.TQ_PROD, 2, seed_rotation=573, seed_sketch=574)
    codec = o.turboquant_codec(D, 2, "prod", rot_seed=573, sketch_seed=574)
    buf, encs = synthetic_db(codec, n, 575)
    q = synth.lowrank_vectors(8, synth.LowRankLaw(D, 64, 576), 577)
    s, i = tq.search_topk(cb, q.to(DEV), up(buf), n, k)
    s, i = s.cpu().numpy(), i.cpu().numpy()
    full = oracle_scores(codec, q.double().numpy(), encs)
    rs, ri = o.topk(full, k)
    for r in range(q.shape[0]):
        tol = 1e-3 * np.linalg.norm(q[r].numpy())
        near = np.abs(full[r] - rs[r, -1]) <= tol
        diff = set(i[r].tolist()) ^ set(ri[r].tolist())
        assert all(near[j] for j in diff), f"query {r}: top-k differs beyond near-ties"
        assert np.all(np.diff(s[r]) <= 0)
        assert np.all(np.abs(s[r] - full[r, i[r]]) <= tol)
