"""Query sets larger than one internal pass of tq_score (261632 queries) and
tq_search_topk (65408 queries): the library runs consecutive passes over
blocks of queries that share one workspace.  Rows on both sides of every
pass boundary are checked against the oracle ([TQ] paper review, "Method"
for the scores; "Validation" for the search over the codes)."""
import sys

import numpy as np
import pytest
import torch

import kv_cache_compression_encode_amd as tq
import synth
from oracle import tq_oracle as o
from tests.parity import check_scores

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOPK_PASS = 65408
SCORE_PASS = 4 * TOPK_PASS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def up(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def _sample_rows(nq, pass_rows):
    rows = {0, 1, nq - 1}
    for b in range(pass_rows, nq, pass_rows):
        rows |= {b - 1, b, b + 1}
    return sorted(r for r in rows if 0 <= r < nq)


@pytest.mark.parametrize("mode,bits", [("prod", 3), ("mse", 4)])
def test_topk_more_queries_than_one_pass(mode, bits):
    # prod b = 3 takes the MFMA search kernel, mse b = 4 the general path
    # (dense score chunks, segment lists, merge)
    n, k = 2048, 10
    nq = TOPK_PASS + 300
    say(f"top-k over {nq} queries ({mode} b={bits})")
    x = synth.iid_gaussian(n, 128, 61)
    q = synth.iid_gaussian(nq, 128, 62)
    if mode == "prod":
        cb = tq.Codebook(128, tq.TQ_PROD, bits, seed_rotation=63, seed_sketch=64)
        codec = o.turboquant_codec(128, bits, "prod", rot_seed=63, sketch_seed=64)
    else:
        cb = tq.Codebook(128, tq.TQ_MSE, bits, seed_rotation=63)
        codec = o.turboquant_codec(128, bits, "mse", rot_seed=63)
    ref = o.encode(codec, x.double().numpy())
    s, i = tq.search_topk(cb, q.to(DEV), up(o.pack(codec, ref)), n, k)
    s, i = s.cpu().numpy(), i.cpu().numpy()
    rows = _sample_rows(nq, TOPK_PASS)
    full = o.score(codec, q[rows].double().numpy(), ref)
    rs, ri = o.topk(full, k)
    nx = ref.nx.astype(np.float64)
    for r, row in enumerate(rows):
        tol = 1e-3 * np.linalg.norm(q[row].numpy()) * nx
        kth = rs[r, -1]
        diff = set(i[row].tolist()) ^ set(ri[r].tolist())
        assert all(abs(full[r, j] - kth) <= 2 * tol[j] for j in diff), f"query {row}: top-k differs beyond near-ties"
        assert np.all(np.abs(s[row] - full[r, i[row]]) <= tol[i[row]]), f"query {row}: scores"
    say(f"checked rows {rows}")


def test_score_more_queries_than_one_pass():
    n = 64
    nq = SCORE_PASS + 200
    say(f"scores of {nq} queries x {n} keys")
    x = synth.iid_gaussian(n, 128, 71)
    q = synth.iid_gaussian(nq, 128, 72)
    cb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=73, seed_sketch=74)
    codec = o.turboquant_codec(128, 3, "prod", rot_seed=73, sketch_seed=74)
    ref = o.encode(codec, x.double().numpy())
    got = tq.score(cb, q.to(DEV), up(o.pack(codec, ref)), n).cpu().numpy()
    rows = _sample_rows(nq, SCORE_PASS)
    qs = q[rows].numpy()
    say("max scaled error", check_scores(got[rows], o.score(codec, q[rows].double().numpy(), ref), qs, ref.nx))
