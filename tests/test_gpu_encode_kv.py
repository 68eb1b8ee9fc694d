"""tq_encode_kv (keys and values of the same tokens in one call) on the
MI355X: its records equal those of the two tq_encode calls byte for byte,
whether the pair runs as one launch or falls back to two, and they match the
oracle.  Every call goes through the C ABI via the thin binding."""
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


def gqa_codecs(**kw):
    kcb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=203, seed_sketch=204, **kw)
    vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=213, layout=tq.TQ_LAYOUT_COL, **kw)
    return kcb, vcb


def both_ways(kcb, vcb, K, V):
    """(paired records, single-call records) for keys and values, as numpy."""
    kr, vr = tq.encode_kv(kcb, vcb, K, V)
    k1, v1 = tq.encode(kcb, K), tq.encode(vcb, V)
    torch.cuda.synchronize()
    return kr.cpu().numpy(), vr.cpu().numpy(), k1.cpu().numpy(), v1.cpu().numpy()


def test_encode_kv_gqa_layer_one_launch():
    # the full decode layer's K and V (8 heads x 32768 bf16 tokens): the pair
    # that runs as one launch; byte-identical to the single encodes, and two
    # heads against the oracle
    Hkv, T = 8, 32768
    say("encode_kv: GQA layer, 8 x 32768 bf16")
    law = synth.KVLaw(Hkv, 128, 205)
    K = synth.kv_cache(1, Hkv, T, 128, 201, law, device=DEV)[0]
    V = synth.kv_cache(1, Hkv, T, 128, 251, law, device=DEV)[0]
    kcb, vcb = gqa_codecs()
    kr, vr, k1, v1 = both_ways(kcb, vcb, K, V)
    assert np.array_equal(kr, k1)
    assert np.array_equal(vr, v1)
    kc = o.turboquant_codec(128, 3, "prod", rot_seed=203, sketch_seed=204)
    vc = o.turboquant_codec(128, 4, "mse", rot_seed=213, layout="col")
    per_k, per_v = kcb.records_bytes(T), vcb.records_bytes(T)
    for h in (0, Hkv - 1):
        xk = K[h, :4096].float().cpu().double().numpy()
        xv = V[h, :4096].float().cpu().double().numpy()
        nb_k, nb_v = kcb.records_bytes(4096), vcb.records_bytes(4096)
        check_encoded(kc, o.encode(kc, xk), o.unpack(kc, kr[h * per_k:h * per_k + nb_k], 4096))
        check_encoded(vc, o.encode(vc, xv), o.unpack(vc, vr[h * per_v:h * per_v + nb_v], 4096))


@pytest.mark.parametrize("B,H,T", [(2, 3, 1000), (1, 1, 1), (3, 5, 65), (1, 16, 200)])
def test_encode_kv_ragged_strided(B, H, T):
    # ragged token counts (a partial last tile), several sequences and heads,
    # rows read through strides (a slice of a wider buffer)
    say(f"encode_kv: B={B} H={H} T={T}, strided bf16")
    g = torch.Generator().manual_seed(B * 1000 + H * 10 + T)
    wide = torch.randn(B, H, T, 256, generator=g).to(torch.bfloat16).to(DEV)
    K, V = wide[..., :128], wide[..., 128:]
    kcb, vcb = gqa_codecs()
    kr, vr, k1, v1 = both_ways(kcb, vcb, K, V)
    assert np.array_equal(kr, k1)
    assert np.array_equal(vr, v1)


@pytest.mark.parametrize("case", ["fp32", "keys_b2", "values_row", "hadamard"])
def test_encode_kv_two_launch_pairs(case):
    # pairs outside the one-launch kernel run as the two encodes
    say(f"encode_kv: fallback pair {case}")
    g = torch.Generator().manual_seed(7)
    K = torch.randn(2, 300, 128, generator=g)
    V = torch.randn(2, 300, 128, generator=g)
    if case != "fp32":
        K, V = K.to(torch.bfloat16), V.to(torch.bfloat16)
    K, V = K.to(DEV), V.to(DEV)
    if case == "keys_b2":
        kcb = tq.Codebook(128, tq.TQ_PROD, 2, seed_rotation=5, seed_sketch=6)
        vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=7, layout=tq.TQ_LAYOUT_COL)
    elif case == "values_row":
        kcb = tq.Codebook(128, tq.TQ_PROD, 3, seed_rotation=5, seed_sketch=6)
        vcb = tq.Codebook(128, tq.TQ_MSE, 4, seed_rotation=7)
    elif case == "hadamard":
        kcb, vcb = gqa_codecs(rotation=tq.TQ_ROT_HADAMARD)
    else:
        kcb, vcb = gqa_codecs()
    kr, vr, k1, v1 = both_ways(kcb, vcb, K, V)
    assert np.array_equal(kr, k1)
    assert np.array_equal(vr, v1)


def test_encode_kv_many_sets():
    # 2 x 32800 (sequence, head) sets of one token: the one-launch grid holds
    # 131200 workgroups along x; every set against the single encodes
    B, H = 2, 32800
    say(f"encode_kv: {B} x {H} sets of one token")
    g = torch.Generator().manual_seed(23)
    K = torch.randn(B, H, 1, 128, generator=g).to(torch.bfloat16).to(DEV)
    V = torch.randn(B, H, 1, 128, generator=g).to(torch.bfloat16).to(DEV)
    kcb, vcb = gqa_codecs()
    kr, vr, k1, v1 = both_ways(kcb, vcb, K, V)
    assert np.array_equal(kr, k1)
    assert np.array_equal(vr, v1)
