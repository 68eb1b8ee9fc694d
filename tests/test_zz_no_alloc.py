"""The decode entry point that allocates nothing (its workspace is the
library's device array) against tq_decode_attend with a caller workspace, on
two calls in a row, the second smaller (MI355X)."""
import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_compression_encode_amd as tq
from kv_cache_compression_encode_amd import _lib as L
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(kcb, vcb, B, Hq, Hkv, T, seq_lens, seed):
    law = synth.KVLaw(Hkv, 128, seed)
    K = synth.kv_cache(B, Hkv, T, 128, seed + 1, law, device=DEV)
    V = synth.kv_cache(B, Hkv, T, 128, seed + 2, law, device=DEV)
    q = synth.kv_queries(B, Hq, Hkv, 128, seed + 3, law, device=DEV)
    krec, vrec = tq.encode(kcb, K), tq.encode(vcb, V)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(128)
    ref = tq.decode_attend(kcb, vcb, q, krec, vrec, T, Hkv, scale, seq_lens=sl)
    out = torch.full_like(ref, float("nan"))
    tq.decode_attend_noalloc(kcb, vcb, q, krec, vrec, T, Hkv, scale, out, seq_lens=sl)
    torch.cuda.synchronize()
    nvmax = float(torch.max(torch.abs(V.float())).item()) * math.sqrt(128)
    err = float(torch.max(torch.abs(out - ref)).item())
    say(f"B={B} Hq={Hq} Hkv={Hkv} T={T}: max |noalloc - workspace| = {err:.3g} "
        f"(bit-identical: {bool(torch.equal(out, ref))})")
    assert torch.isfinite(out).all()
    assert err <= 1e-3 * nvmax
    return out, ref


def test_noalloc_decode_matches_workspace_decode_twice():
    kcb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=203, seed_sketch=204)
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=207, layout=tq.TQ_LAYOUT_COL)
    # first call: 2 sequences x 8 query heads over 2 KV heads, 5000 tokens
    _case(kcb, vcb, 2, 8, 2, 5000, [5000, 1777], 811)
    # second call, smaller: the shared array keeps the first call's contents
    _case(kcb, vcb, 1, 4, 1, 300, [300], 821)


def test_noalloc_decode_rejects_oversize():
    kcb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=203, seed_sketch=204)
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=207, layout=tq.TQ_LAYOUT_COL)
    B, Hq, Hkv, T = 64, 32, 8, 65536
    need = kcb.workspace(L.TQ_OP_DECODE, B * Hq, T, Hkv)
    assert need > L.TQ_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, Hq, 128, device=DEV)
    rec = torch.zeros(16, dtype=torch.uint8, device=DEV)
    out = torch.zeros(B, Hq, 128, device=DEV)
    with pytest.raises(tq.TQError) as e:
        tq.decode_attend_noalloc(kcb, vcb, q, rec, rec, T, Hkv, 0.1, out)
    assert e.value.status == L.TQ_EWORKSPACE
