"""Benchmark of the compressed-KV hot path on one MI355X.

Default workload (one step): one decode layer shaped like an 8B GQA model --
32 query heads over 8 KV heads, head dim 128, 32768 cached tokens, batch 1,
bf16 keys/values from the anisotropic synthetic law.  A step encodes the
layer's keys (TurboQuant-prod, 3 bits) and values (TurboQuant-mse, 4 bits)
in one tq_encode_kv call, then runs one fused decode-attention step (score 32 queries against the
compressed keys, softmax, .V over the compressed values).  Steps and the
per-call timings cycle over 16 distinct layers (2.1 GB of bf16 inputs, 495 MB
of records), more than the 256 MB Infinity Cache holds, so every call streams
its inputs from HBM.  Reported value: keys per second through the whole step.

Other workloads (--workload): gqa_outlier (the same layer with 2.5-bit
outlier-split keys: per KV head the 32 largest-RMS channels at 3 bits, the
other 96 at 2 bits, two TurboQuant instances), gqa_outlier_kv (2.5-bit split
keys and values), small (4096 fp32 vectors, 16 queries),
bulk_prefill (32 layers x 8 heads x 131072 tokens), sq_decode (SpectralQuant
keys, 64 sequences x 8192 tokens), vector_search (1e6 x 1536 database, 1024
queries, top-10).  Each prints one JSON line of the same shape.

Per-call HIP-event timings (on the stream the library launches on) give the
achieved GB/s or TFLOP/s of each call; the dominant one goes in "roofline".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
D, HQ, HKV, T = 128, 32, 8, 32768
NLAYERS = 16
# Algorithmic bytes per vector: input row + record bytes (codes, signs, fp16 norms).
K_REC, V_REC = 52, 66
K_REC_SPLIT = 44                     # split keys: 16 + 4 code bytes, 16 sign bytes, 4 fp16 norms
V_REC_SPLIT = 40                     # split values: 16 + 16 + 4 code bytes, 2 fp16 norms
K_ENC_BYTES = 2 * D + K_REC          # 308 B per key
V_ENC_BYTES = 2 * D + V_REC          # 322 B per value
DEC_BYTES = K_REC + V_REC            # 118 B per cached token-head read by decode
# HBM bytes per launch of a call's kernel from rocprofv3 FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch), each scaled by what the counter reads for a
# plain 1 GiB device copy (factors 2.0 and 1.0); the summary and the commands
# are in profiles/.  Keyed by (workload, call): a reading holds for that
# launch size only, and for the kernels as built when the counters were
# taken; a pair missing here reports null.
TRAFFIC = {("gqa_layer", "encode_kv"): 176005564, ("gqa_layer", "encode_keys"): 82160425,
           ("gqa_layer", "encode_values"): 93543491}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="gqa_layer",
                   choices=["gqa_layer", "gqa_outlier", "gqa_outlier_kv", "small", "bulk_prefill", "sq_decode",
                            "vector_search"])
    p.add_argument("--bits", type=int, default=2, help="vector_search: TurboQuant-prod bits (2 or 4)")
    p.add_argument("--rotation", default="haar", choices=["haar", "hadamard"],
                   help="gqa_layer / bulk_prefill: dense seeded Haar Pi (default) or the randomized "
                        "Hadamard rotation mode")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", action="store_true",
                   help="run only a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


def copy_probe():
    import torch
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": a.numel() * 4}), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] + [1]))
    except Exception:
        return os.cpu_count() or 1


def _time_loop(fn, budget_s=10.0, max_reps=100000):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el > budget_s or reps >= max_reps:
            return reps, el


# ------------------------------------------------------------ oracle legs
def cpu_baseline_gqa():
    """The oracle on a bounded sample: one KV head, 4096 tokens, encode of K
    and V then the 4 query heads' decode step."""
    import synth
    from oracle import tq_oracle as o
    n = 4096
    law = synth.KVLaw(1, D, 205)
    k = synth.kv_cache(1, 1, n, D, 201, law)[0, 0].double().numpy()
    v = synth.kv_cache(1, 1, n, D, 251, law)[0, 0].double().numpy()
    q = synth.kv_queries(1, 4, 1, D, 202, law)[0].double().numpy()
    kc = o.turboquant_codec(D, 3, "prod", rot_seed=203, sketch_seed=204, rotation=ROTATION)
    vc = o.turboquant_codec(D, 4, "mse", rot_seed=203, layout="col", rotation=ROTATION)

    def run():
        ke, ve = o.encode(kc, k), o.encode(vc, v)
        o.decode_attention(kc, vc, q, [ke], [ve], 1 / math.sqrt(D))
    reps, el = _time_loop(run)
    return {"value": reps * n / el, "unit": "keys/s", "cores": _cores(), "kind": "oracle",
            "sample": f"1 kv head x {n} tokens (encode K+V, 4-head decode), {reps} reps in {el:.1f} s"}


def outlier_channels(torch, law, heads, o_=32, n=2048, seed=900):
    """Per KV head the o_ channels of largest RMS over n calibration tokens
    (the split's channel lists, found once before the cache is built)."""
    import numpy as np
    out = []
    for h in range(heads):
        x = law.sample(h, n, torch.Generator().manual_seed(seed + h), "cpu").double()
        out.append(np.argsort(-x.pow(2).mean(dim=0).sqrt().numpy(), kind="stable")[:o_])
    return np.stack(out).astype(np.int32)


def cpu_baseline_gqa_outlier():
    """The oracle on a bounded sample: one KV head, 4096 tokens, split encode
    of K, encode of V, then the 4 query heads' decode step."""
    import torch
    import synth
    from oracle import tq_oracle as o
    n = 4096
    law = synth.KVLaw(1, D, 205)
    k = synth.kv_cache(1, 1, n, D, 201, law)[0, 0].double().numpy()
    v = synth.kv_cache(1, 1, n, D, 251, law)[0, 0].double().numpy()
    q = synth.kv_queries(1, 4, 1, D, 202, law)[0].double().numpy()
    kc = o.outlier_split_codec(D, outlier_channels(torch, law, 1), 3, 2, "prod", rot_seed=203, sketch_seed=204)
    vc = o.turboquant_codec(D, 4, "mse", rot_seed=203, layout="col")

    def run():
        ke, ve = o.split_encode(kc, k), o.encode(vc, v)
        o.split_decode_attention(kc, vc, q, [ke], [ve], 1 / math.sqrt(D))
    reps, el = _time_loop(run)
    return {"value": reps * n / el, "unit": "keys/s", "cores": _cores(), "kind": "oracle",
            "sample": f"1 kv head x {n} tokens (split encode K, encode V, 4-head decode), {reps} reps in {el:.1f} s"}


def cpu_baseline_gqa_outlier_kv():
    """The oracle on a bounded sample: one KV head, 4096 tokens, split encode
    of K and of V, then the 4 query heads' decode step."""
    import torch
    import synth
    from oracle import tq_oracle as o
    n = 4096
    law = synth.KVLaw(1, D, 205)
    k = synth.kv_cache(1, 1, n, D, 201, law)[0, 0].double().numpy()
    v = synth.kv_cache(1, 1, n, D, 251, law)[0, 0].double().numpy()
    q = synth.kv_queries(1, 4, 1, D, 202, law)[0].double().numpy()
    ch = outlier_channels(torch, law, 1)
    kc = o.outlier_split_codec(D, ch, 3, 2, "prod", rot_seed=203, sketch_seed=204)
    vc = o.outlier_split_codec(D, ch, 3, 2, "mse", rot_seed=213, layout="col")

    def run():
        ke, ve = o.split_encode(kc, k), o.split_encode(vc, v)
        o.split_decode_attention(kc, vc, q, [ke], [ve], 1 / math.sqrt(D))
    reps, el = _time_loop(run)
    return {"value": reps * n / el, "unit": "keys/s", "cores": _cores(), "kind": "oracle",
            "sample": f"1 kv head x {n} tokens (split encode K and V, 4-head decode), {reps} reps in {el:.1f} s"}


def cpu_baseline_small():
    import synth
    from oracle import tq_oracle as o
    x = synth.iid_gaussian(4096, D, synth.seed(1, "data")).double().numpy()
    q = synth.iid_gaussian(16, D, synth.seed(1, "queries")).double().numpy()
    c = o.turboquant_codec(D, 3, "prod", rot_seed=103, sketch_seed=104)

    def run():
        o.score(c, q, o.encode(c, x))
    reps, el = _time_loop(run)
    return {"value": reps * 4096 / el, "unit": "vectors/s", "cores": _cores(), "kind": "oracle",
            "sample": f"the whole workload (encode 4096 + score 16 x 4096), {reps} reps in {el:.1f} s"}


def cpu_baseline_bulk():
    import synth
    from oracle import tq_oracle as o
    n = 4096
    law = synth.KVLaw(1, D, 305)
    k = synth.kv_cache(1, 1, n, D, 301, law)[0, 0].double().numpy()
    v = synth.kv_cache(1, 1, n, D, 306, law)[0, 0].double().numpy()
    kc = o.turboquant_codec(D, 3, "prod", rot_seed=303, sketch_seed=304, rotation=ROTATION)
    vc = o.turboquant_codec(D, 4, "mse", rot_seed=303, layout="col", rotation=ROTATION)

    def run():
        o.pack(kc, o.encode(kc, k))
        o.pack(vc, o.encode(vc, v))
    reps, el = _time_loop(run)
    return {"value": reps * n / el, "unit": "token-heads/s", "cores": _cores(), "kind": "oracle",
            "sample": f"1 head x {n} tokens, encode+pack of K and V, {reps} reps in {el:.1f} s"}


def cpu_baseline_sq():
    import numpy as np
    import torch
    import synth
    from oracle import tq_oracle as o
    n = 8192
    law = synth.KVLaw(1, D, 405)
    k = synth.kv_cache(1, 1, n, D, 401, law)[0, 0].double().numpy()
    v = synth.kv_cache(1, 1, n, D, 406, law)[0, 0].double().numpy()
    q = synth.kv_queries(1, 4, 1, D, 402, law)[0].double().numpy()
    calib = law.sample(0, 2048, torch.Generator().manual_seed(405), "cpu").float().numpy()
    kc = o.spectralquant_codec(calib.astype(np.float64)[None], [5, 3, 2, 2] + [1] * 124, 4,
                               sketch_seed=404)
    vc = o.turboquant_codec(D, 4, "mse", rot_seed=407, layout="col")
    ke, ve = o.encode(kc, k), o.encode(vc, v)

    def run():
        o.decode_attention(kc, vc, q, [ke], [ve], 1 / math.sqrt(D))
    reps, el = _time_loop(run)
    return {"value": reps * n / el, "unit": "token-heads/s", "cores": _cores(), "kind": "oracle",
            "sample": f"1 sequence x 1 kv head x {n} tokens, 4-head decode, {reps} reps in {el:.1f} s"}


def cpu_baseline_search(bits):
    import synth
    from oracle import tq_oracle as o
    n, nq, d = 2048, 1024, 1536
    law = synth.LowRankLaw(d, 64, 505)
    x = synth.lowrank_vectors(n, law, 501).double().numpy()
    q = synth.lowrank_vectors(nq, law, 502).double().numpy()
    c = o.turboquant_codec(d, bits, "prod", rot_seed=503, sketch_seed=504)

    def run():
        o.topk(o.score(c, q, o.encode(c, x)), 10)
    reps, el = _time_loop(run)
    return {"value": reps * n * nq / el, "unit": "query-key pairs/s (incl. encode)", "cores": _cores(),
            "kind": "oracle",
            "sample": f"{n} database vectors x {nq} queries: encode, score, top-10; {reps} reps in {el:.1f} s"}


# ------------------------------------------------------------ timing helpers
def _cycle(fn):
    """A no-argument call cycling fn over the workload's inputs."""
    state = {"i": 0}

    def call():
        fn(state["i"])
        state["i"] += 1
    return call


def time_one(torch, fn, steps, warmup):
    """Average time of `steps` back-to-back calls of fn between one pair of HIP events."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_calls(torch, calls, steps, warmup):
    """Whole-step time, then each call's average launch time.

    calls: list of (name, fn(i)) run in order as one step.  Per call, `steps`
    launches (cycling over the workload's inputs) run back to back between one
    pair of HIP events on torch's current stream, the stream the library
    launches on, so the figure is the kernels' own time plus launch gaps."""
    def step(i):
        for _, fn in calls:
            fn(i)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    per = {}
    for name, fn in calls:
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            fn(i)
        t1.record()
        torch.cuda.synchronize()
        per[name] = t0.elapsed_time(t1) / steps
    return ms_step, per


def result(args, metric, value, unit, ms_step, workload, dtype, roof, breakdown, extra=None):
    res = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": workload,
           "roofline": roof, "breakdown": breakdown}
    if extra:
        res.update(extra)
    return res


ROTATION = "haar"  # set from --rotation


def rot_kw(tq):
    return {"rotation": tq.TQ_ROT_HADAMARD} if ROTATION == "hadamard" else {}


def rot_note(s):
    return s + ("; randomized Hadamard rotation (register Walsh-Hadamard transform in the encode)"
                if ROTATION == "hadamard" else "")


def hbm_roof(workload, name, ms, nbytes, note=None):
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the counters were taken for the dense-Pi kernels
    traffic = TRAFFIC.get((workload, name)) if ROTATION == "haar" else None
    r = {"bound": "hbm", "kernel": name, "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
         "bytes_per_launch": nbytes, "avg_launch_ms": ms}
    if note:
        r["note"] = note
    return r


# ------------------------------------------------------------ workloads
def run_gqa_layer(args, torch, tq, synth, split=False, split_values=False):
    dev = torch.device("cuda:0")
    law = synth.KVLaw(HKV, D, 205)
    K = [synth.kv_cache(1, HKV, T, D, 201 + 1000 * l, law, device=dev)[0] for l in range(NLAYERS)]
    V = [synth.kv_cache(1, HKV, T, D, 251 + 1000 * l, law, device=dev)[0] for l in range(NLAYERS)]
    q = synth.kv_queries(1, HQ, HKV, D, 202, law, device=dev)
    if split:
        # 2.5-bit keys: per KV head 32 outlier channels at 3 bits, 96 at 2 bits
        kcb = tq.Codebook(D, tq.TQ_PROD, 2, seed_rotation=203, seed_sketch=204,
                          outlier_channels=outlier_channels(torch, law, HKV), outlier_bits=3)
    else:
        kcb = tq.Codebook(D, tq.TQ_PROD, 3, seed_rotation=203, seed_sketch=204, **rot_kw(tq))
    if split_values:
        # 2.5-bit values as well: the same channel split, mse, col records
        # (8-token code words that the MFMA decode reads)
        vcb = tq.Codebook(D, tq.TQ_MSE, 2, seed_rotation=213, outlier_channels=outlier_channels(torch, law, HKV),
                          outlier_bits=3, layout=tq.TQ_LAYOUT_COL)
    else:
        vcb = tq.Codebook(D, tq.TQ_MSE, 4, seed_rotation=203, layout=tq.TQ_LAYOUT_COL, **rot_kw(tq))
    k_rec = K_REC_SPLIT if split else K_REC
    v_rec = V_REC_SPLIT if split_values else V_REC
    assert kcb.tile_bytes == 64 * k_rec and vcb.tile_bytes == 64 * v_rec
    krec = [torch.empty(HKV * kcb.records_bytes(T), dtype=torch.uint8, device=dev) for _ in range(NLAYERS)]
    vrec = [torch.empty(HKV * vcb.records_bytes(T), dtype=torch.uint8, device=dev) for _ in range(NLAYERS)]
    out = torch.empty(1, HQ, D, dtype=torch.float32, device=dev)
    ws = tq.DecodeWorkspace(kcb, HQ, T, HKV, dev)
    scale = 1 / math.sqrt(D)

    # the step: keys and values of the layer encoded by one tq_encode_kv call
    # (one launch for this codec pair), then the decode
    calls = [("encode_kv", lambda i: tq.encode_kv(kcb, vcb, K[i % NLAYERS], V[i % NLAYERS],
                                                  krec[i % NLAYERS], vrec[i % NLAYERS])),
             ("decode_attend", lambda i: tq.decode_attend(kcb, vcb, q, krec[i % NLAYERS], vrec[i % NLAYERS], T,
                                                          HKV, scale, out=out, workspace=ws))]
    ms_step, t = time_calls(torch, calls, args.steps, args.warmup)
    # the two encodes as single calls, outside the step
    t1 = {"encode_keys": time_one(torch, _cycle(lambda i: tq.encode(kcb, K[i % NLAYERS], records=krec[i % NLAYERS])),
                                  args.steps, args.warmup),
          "encode_values": time_one(torch, _cycle(lambda i: tq.encode(vcb, V[i % NLAYERS],
                                                                      records=vrec[i % NLAYERS])),
                                    args.steps, args.warmup)}
    # append-on-decode, outside the step: the new token of every KV head
    # encoded into slot T - 1 of the layer's K and V records
    pos = torch.tensor([T - 1], dtype=torch.int32, device=dev)
    kn, vn = K[0][:, T - 1].unsqueeze(0), V[0][:, T - 1].unsqueeze(0)
    append_ms = time_one(torch, lambda: (tq.append(kcb, kn, krec[0], pos, T), tq.append(vcb, vn, vrec[0], pos, T)),
                         args.steps, args.warmup)
    # the whole decode step on a paged view of the same records (pages of 4
    # tiles, the table mapping each KV head to its own pages in order): append
    # the new token at slot T - 1, then attend over T tokens
    page_tiles = 4
    npg = (T // 64) // page_tiles
    table = torch.arange(HKV * npg, dtype=torch.int32, device=dev).reshape(HKV, npg)
    step_ms = time_one(torch, lambda: tq.decode_step(kcb, vcb, q, kn, vn, krec[0], vrec[0], T, HKV, scale, pos,
                                                     out=out, workspace=ws, block_table=table,
                                                     page_tiles=page_tiles),
                       args.steps, args.warmup)
    nk = HKV * T
    nbytes = {"encode_keys": nk * (2 * D + k_rec), "encode_values": nk * (2 * D + v_rec),
              "encode_kv": nk * (4 * D + k_rec + v_rec), "decode_attend": nk * (k_rec + v_rec)}
    dom = max(t, key=lambda k: t[k])
    tall = {**t, **t1}
    bd = {k: {"ms": tall[k], "GBps": nbytes[k] / (tall[k] * 1e-3) / 1e9,
              "hbm_frac": nbytes[k] / (tall[k] * 1e-3) / 1e9 / HBM_PEAK_GBS} for k in tall}
    keys_desc = ("K outlier-channel split, 2.5 bits (per KV head the 32 largest-RMS channels of a 2048-token "
                 "calibration sample: TurboQuant-prod b=3; the other 96: b=2; row records, 44 B/key)"
                 if split else "K TurboQuant-prod b=3 (row records)")
    vals_desc = ("V outlier-channel split, 2.5 bits (the same channels: TurboQuant-mse b=3 on them, b=2 "
                 "on the other 96; col records, 40 B/value)"
                 if split_values else "V TurboQuant-mse b=4 (col records)")
    wname = "gqa_outlier_kv" if split_values else ("gqa_outlier" if split else "gqa_layer")
    roof = hbm_roof(wname, dom, t[dom], nbytes[dom])
    res = result(args, "compressed-key scoring keys/s & KV encode GB/s at d=128, % of HBM roofline",
                 nk / (ms_step * 1e-3), "keys/s", ms_step,
                 {"workload": rot_note(("gqa_decode_layer" if wname == "gqa_layer" else wname) +
                                       ": 32 q / 8 kv heads, d=128, 32768 tokens, batch 1, "
                                       f"bf16 K/V; {keys_desc}, {vals_desc}; step = encode K and V "
                                       "(one tq_encode_kv call) + decode attention"),
                  "layers_cycled": NLAYERS},
                 "f32 (split-f16 MFMA)", roof, bd,
                 {"decode_keys_per_s": nk / (t["decode_attend"] * 1e-3),
                  "append_kv_ms": append_ms,
                  "decode_step_paged_ms": step_ms,
                  "encode_GBps": nbytes["encode_kv"] / (t["encode_kv"] * 1e-3) / 1e9})
    if split_values:
        return res, cpu_baseline_gqa_outlier_kv
    return res, (cpu_baseline_gqa_outlier if split else cpu_baseline_gqa)


def run_small(args, torch, tq, synth):
    dev = torch.device("cuda:0")
    n, nq = 4096, 16
    x = synth.iid_gaussian(n, D, synth.seed(1, "data"), device=dev)
    q = synth.iid_gaussian(nq, D, synth.seed(1, "queries"), device=dev)
    cb = tq.Codebook(D, tq.TQ_PROD, 3, seed_rotation=103, seed_sketch=104)
    rec = torch.empty(cb.records_bytes(n), dtype=torch.uint8, device=dev)

    calls = [("encode", lambda i: tq.encode(cb, x, records=rec)),
             ("score", lambda i: tq.score(cb, q, rec, n))]
    ms_step, t = time_calls(torch, calls, args.steps, args.warmup)
    nbytes = {"encode": n * (4 * D + 52), "score": n * 52 + nq * n * 4}
    bd = {k: {"ms": t[k], "GBps": nbytes[k] / (t[k] * 1e-3) / 1e9} for k in t}
    res = result(args, "TurboQuant-prod encode + score vectors/s (d=128, 4096 vectors, 16 queries)",
                 n / (ms_step * 1e-3), "vectors/s", ms_step,
                 {"workload": "small: 4096 iid N(0,I) fp32 vectors d=128, prod b=3, encode then "
                              "score 16 queries x 4096 keys"},
                 "f32 (split-f16 MFMA)",
                 hbm_roof("small", "encode", t["encode"], nbytes["encode"],
                          "2 MiB workload: launch-bound, cache-resident; fraction shown for completeness"),
                 bd, {"score_keys_per_s": n * nq / (t["score"] * 1e-3)})
    return res, cpu_baseline_small


def run_bulk(args, torch, tq, synth):
    dev = torch.device("cuda:0")
    L, H, TT = 32, 8, 131072
    law = synth.KVLaw(H, D, 305)
    K = synth.kv_cache(L, H, TT, D, 301, law, device=dev)
    V = synth.kv_cache(L, H, TT, D, 306, law, device=dev)
    kcb = tq.Codebook(D, tq.TQ_PROD, 3, seed_rotation=303, seed_sketch=304, **rot_kw(tq))
    vcb = tq.Codebook(D, tq.TQ_MSE, 4, seed_rotation=303, layout=tq.TQ_LAYOUT_COL, **rot_kw(tq))
    krec = torch.empty(L * H * kcb.records_bytes(TT), dtype=torch.uint8, device=dev)
    vrec = torch.empty(L * H * vcb.records_bytes(TT), dtype=torch.uint8, device=dev)

    # the step: one tq_encode_kv call (one launch for this codec pair)
    calls = [("encode_kv", lambda i: tq.encode_kv(kcb, vcb, K, V, krec, vrec))]
    ms_step, t = time_calls(torch, calls, args.steps, args.warmup)
    # the two encodes as single calls, outside the step
    t1 = {"encode_keys": time_one(torch, lambda: tq.encode(kcb, K, records=krec), args.steps, args.warmup),
          "encode_values": time_one(torch, lambda: tq.encode(vcb, V, records=vrec), args.steps, args.warmup)}
    nk = L * H * TT
    nbytes = {"encode_keys": nk * K_ENC_BYTES, "encode_values": nk * V_ENC_BYTES,
              "encode_kv": nk * (K_ENC_BYTES + V_ENC_BYTES)}
    dom = max(t, key=lambda k: t[k])
    tall = {**t, **t1}
    bd = {k: {"ms": tall[k], "GBps": nbytes[k] / (tall[k] * 1e-3) / 1e9,
              "hbm_frac": nbytes[k] / (tall[k] * 1e-3) / 1e9 / HBM_PEAK_GBS} for k in tall}
    gbs = nbytes["encode_kv"] / (ms_step * 1e-3) / 1e9
    res = result(args, "KV encode GB/s at d=128 (bulk prefill), % of HBM roofline", gbs, "GB/s", ms_step,
                 {"workload": rot_note("bulk_prefill: 32 layers x 8 kv heads x 131072 tokens x d=128 bf16 K "
                                       "and V; K prod b=3 row, V mse b=4 col; step = encode all K and V "
                                       "(one tq_encode_kv call)")},
                 "f32 (split-f16 MFMA)", hbm_roof("bulk_prefill", dom, t[dom], nbytes[dom]), bd,
                 {"token_heads_per_s": nk / (ms_step * 1e-3),
                  "compression_ratio": (2 * D * 2) / (K_REC + V_REC)})
    return res, cpu_baseline_bulk


def run_sq(args, torch, tq, synth):
    dev = torch.device("cuda:0")
    B, H, TT, QH = 64, 8, 8192, 32
    law = synth.KVLaw(H, D, 405)
    calib = torch.stack([law.sample(h, 2048, torch.Generator().manual_seed(405 + h), "cpu")
                         for h in range(H)])
    # calibration pass (the pages put theirs at 15 s per model): per-head
    # moments of the calibration keys on the GPU (fp64), then the eigenbases,
    # per-dim scales and codebooks on host threads; the all-host build beside it
    calib_dev = calib.to(dev)
    torch.cuda.synchronize()
    kw = dict(bitmap=[5, 3, 2, 2] + [1] * 124, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE, num_heads=H,
              seed_sketch=404)
    t_cal = time.perf_counter()
    kcb = tq.Codebook(D, tq.TQ_PROD, 0, calib=calib_dev, **kw)
    calib_s = time.perf_counter() - t_cal
    t_cal = time.perf_counter()
    tq.Codebook(D, tq.TQ_PROD, 0, calib=calib, **kw)
    calib_host_s = time.perf_counter() - t_cal
    del calib_dev
    # the map water-filling would pick from this spectrum at the same budget
    wf = tq.Codebook(D, tq.TQ_PROD, 0, qjl_dims=4, rotation=tq.TQ_ROT_CALIBRATE, num_heads=H,
                     seed_sketch=404, calib=calib, waterfill_bits=136, device=-1)
    wf_bits = [int(v).bit_length() - 1 for v in wf.export(0)[4][:8]]
    vcb = tq.Codebook(D, tq.TQ_MSE, 4, seed_rotation=407, layout=tq.TQ_LAYOUT_COL)
    ncache = 2
    krec, vrec, qs = [], [], []
    for c in range(ncache):
        K = synth.kv_cache(B, H, TT, D, 401 + 10 * c, law, device=dev)
        krec.append(tq.encode(kcb, K))
        del K
        V = synth.kv_cache(B, H, TT, D, 406 + 10 * c, law, device=dev)
        vrec.append(tq.encode(vcb, V))
        del V
        qs.append(synth.kv_queries(B, QH, H, D, 402 + 10 * c, law, device=dev))
    torch.cuda.synchronize()
    kper, vper = kcb.records_bytes(TT), vcb.records_bytes(TT)
    out = torch.empty(B, QH, D, dtype=torch.float32, device=dev)
    ws = tq.DecodeWorkspace(kcb, B * QH, TT, H, dev)
    scale = 1 / math.sqrt(D)

    calls = [("decode_attend", lambda i: tq.decode_attend(kcb, vcb, qs[i % ncache], krec[i % ncache],
                                                          vrec[i % ncache], TT, H, scale, out=out, workspace=ws))]
    ms_step, t = time_calls(torch, calls, args.steps, args.warmup)
    # append-on-decode, outside the step: one new K and V token per sequence
    # and KV head into slot TT - 1
    pos = torch.full((B,), TT - 1, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev).manual_seed(409)
    kn = torch.randn(B, H, D, generator=gen, device=dev).to(torch.bfloat16)
    vn = torch.randn(B, H, D, generator=gen, device=dev).to(torch.bfloat16)
    append_ms = time_one(torch, lambda: (tq.append(kcb, kn, krec[0], pos, TT), tq.append(vcb, vn, vrec[0], pos, TT)),
                         args.steps, args.warmup)
    # the SpectralQuant key encode of one cache, outside the step
    K = synth.kv_cache(B, H, TT, D, 401, law, device=dev)
    enc_ms = time_one(torch, lambda: tq.encode(kcb, K, records=krec[0]), 5, 1)
    del K
    nk = B * H * TT
    nbytes = nk * (kper + vper) // TT
    res = result(args, "SpectralQuant batched decode token-heads/s, % of HBM roofline",
                 nk / (ms_step * 1e-3), "token-heads/s", ms_step,
                 {"workload": "sq_decode: 64 sequences x 8192 tokens, 8 kv / 32 q heads, d=128; keys "
                              "SpectralQuant (per-head eigenbasis, bits [5,3,2,2]+1, QJL on 4 dims), "
                              "values mse b=4 col; step = one fused decode token per sequence",
                  "caches_cycled": ncache},
                 "f32", hbm_roof("sq_decode", "decode_attend", t["decode_attend"], nbytes,
                                 "one library call: the fused score + softmax + P V kernel, which rotates its "
                                 "queries in its set-up; one split per sequence at this batch, so the merge "
                                 "and the inverse value rotation run inside it"),
                 {"decode_attend": {"ms": t["decode_attend"], "bytes": nbytes}},
                 {"record_bytes_per_token_head": (kper + vper) / TT,
                  "append_kv_ms": append_ms,
                  "encode_keys_ms": enc_ms,
                  "encode_keys_GBps": nk * (2 * D + kper / TT) / (enc_ms * 1e-3) / 1e9,
                  "calibration_s": calib_s,
                  "calibration_host_s": calib_host_s,
                  "calibration": "8 heads x 2048 tokens: moments on the GPU (fp64), then per head on host "
                                 "threads the Jacobi eigenbasis, per-dim "
                                 "scales, Lloyd-Max codebooks, device upload",
                  "waterfill_bits_dims0to7_at_136": wf_bits})
    return res, cpu_baseline_sq


def run_search(args, torch, tq, synth):
    dev = torch.device("cuda:0")
    n, nq, d, k = 1_000_000, 1024, 1536, 10
    law = synth.LowRankLaw(d, 64, 505, device=dev)
    x = synth.lowrank_vectors(n, law, 501, device=dev)
    q = synth.lowrank_vectors(nq, law, 502, device=dev)
    cb = tq.Codebook(d, tq.TQ_PROD, args.bits, seed_rotation=503, seed_sketch=504)
    rec = torch.empty(cb.records_bytes(n), dtype=torch.uint8, device=dev)

    calls = [("encode", lambda i: tq.encode(cb, x, records=rec)),
             ("search_topk", lambda i: tq.search_topk(cb, q, rec, n, k))]
    ms_step, t = time_calls(torch, calls, args.steps, args.warmup)
    m = d
    flops = {"encode": n * 2 * (d * d + m * m), "search_topk": 2 * nq * n * (d + m)}
    tf = {kk: flops[kk] / (t[kk] * 1e-3) / 1e12 for kk in t}
    dom = max(t, key=lambda kk: t[kk])
    roof = {"bound": "mfma", "kernel": dom, "achieved": tf[dom], "peak": 2500.0, "unit": "TFLOP/s",
            "frac": tf[dom] / 2500.0, "traffic": None, "flops_per_launch": flops[dom],
            "avg_launch_ms": t[dom],
            "note": "algorithmic flops (one pass per product) over the call's duration; the GEMMs "
                    "run in fp16 on MFMA (peak 2.5 PFLOP/s) with hi/lo splits for fp32 accuracy"}
    bd = {kk: {"ms": t[kk], "TFLOPs": tf[kk], "mfma_frac": tf[kk] / 2500.0} for kk in t}
    # recall@10 of all 1024 queries against the exact top-10 of <q, x>,
    # outside the timed region: fp64 products in chunks with torch (nothing
    # shared with the library's kernels)
    s_top, i_top = tq.search_topk(cb, q, rec, n, k)
    torch.cuda.synchronize()
    qd = q.double()
    best_s = torch.full((nq, k), -float("inf"), dtype=torch.float64, device=dev)
    best_i = torch.zeros((nq, k), dtype=torch.int64, device=dev)
    for i0 in range(0, n, 65536):
        sc = qd @ x[i0:i0 + 65536].double().T
        cs, ci = torch.topk(sc, k, dim=1)
        ms, mi = torch.topk(torch.cat([best_s, cs], 1), k, dim=1)
        best_i = torch.gather(torch.cat([best_i, ci + i0], 1), 1, mi)
        best_s = ms
    hits = (i_top.unsqueeze(2) == best_i.unsqueeze(1)).any(dim=2).sum().item()
    recall = hits / (nq * k)
    res = result(args, f"vector search (d=1536, prod b={args.bits}): query-key pairs/s incl. encode",
                 nq * n / (ms_step * 1e-3), "pairs/s", ms_step,
                 {"workload": f"vector_search: 1e6 x 1536 fp32 unit vectors (rank-64 half energy), "
                              f"TurboQuant-prod b={args.bits}; step = encode database + top-10 of "
                              f"1024 queries"},
                 "f32 (split-f16 MFMA)", roof, bd,
                 {"encode_vectors_per_s": n / (t["encode"] * 1e-3),
                  "search_pairs_per_s": nq * n / (t["search_topk"] * 1e-3),
                  "recall_at_10": recall,
                  "recall_note": "the returned top-10 of all 1024 queries against the exact top-10 of "
                                 "<q, x> over the 1e6 fp32 vectors (fp64 products)"})
    return res, lambda: cpu_baseline_search(args.bits)


DEFAULT_STEPS = {"gqa_layer": (200, 20), "gqa_outlier": (200, 20), "gqa_outlier_kv": (200, 20), "small": (200, 10),
                 "bulk_prefill": (10, 2),
                 "sq_decode": (200, 20),
                 "vector_search": (3, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): there is no "
              "multi-GPU figure", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    global ROTATION
    ROTATION = args.rotation
    if ROTATION != "haar" and args.workload not in ("gqa_layer", "bulk_prefill"):
        print("--rotation applies to the gqa_layer and bulk_prefill workloads", file=sys.stderr)
        sys.exit(2)
    st, wu = DEFAULT_STEPS[args.workload]
    args.steps = st if args.steps is None else args.steps
    args.warmup = wu if args.warmup is None else args.warmup
    import torch
    import kv_cache_compression_encode_amd as tq
    import synth
    run = {"gqa_layer": run_gqa_layer, "small": run_small,
           "gqa_outlier": lambda *a: run_gqa_layer(*a, split=True),
           "gqa_outlier_kv": lambda *a: run_gqa_layer(*a, split=True, split_values=True), "bulk_prefill": run_bulk,
           "sq_decode": run_sq, "vector_search": run_search}[args.workload]
    res, baseline = run(args, torch, tq, synth)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = baseline()
        res["cpu_baseline"]["cpu"] = _cpu_model()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
