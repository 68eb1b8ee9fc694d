"""Seeded synthetic workloads for the TurboQuant codec.

These generators only draw test and benchmark inputs (vectors, queries,
calibration tokens).  They hold none of the codec's arithmetic: the random
rotation and sketch that the codec itself draws are generated inside the
library and, independently, inside the oracle.

Workloads (sizes and laws):

* ``iid``      -- x ~ N(0, I), fp32 (plain TurboQuant-prod at d=128).
* ``kv``       -- bf16 keys/values of a GQA layer.  Per KV head a zero-mean
  Gaussian whose covariance puts fractions [0.50, 0.16, 0.10, 0.04] of the
  trace into 4 seeded orthonormal directions (about 80 % of the variance in 4 of
  128 dims, with lambda_0 = 0.50 and lambda_3 = 0.04 as in the SpectralQuant
  thread, tweets 2 and 6) and spreads the remaining 0.20 evenly over the
  other 124 directions; trace = d.  Two seeded channels are then scaled by 10.
* ``lowrank``  -- vector-search database: half the energy isotropic, half in a
  seeded rank-64 subspace, each row normalised to unit length, fp32.

All draws use torch generators on the requested device, so a workload is a
pure function of (seed, shapes, device).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

KV_TOP_FRACTIONS = (0.50, 0.16, 0.10, 0.04)
KV_OUTLIER_SCALE = 10.0
KV_NUM_OUTLIERS = 2


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def iid_gaussian(n: int, d: int, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """n x d matrix with i.i.d. N(0, 1) entries."""
    g = _gen(seed, device)
    return torch.randn(n, d, generator=g, device=device, dtype=torch.float32).to(dtype)


def _haar(d: int, k: int, g: torch.Generator, device) -> torch.Tensor:
    """d x k matrix with orthonormal columns drawn from the Haar measure (fp64)."""
    a = torch.randn(d, k, generator=g, device=device, dtype=torch.float64)
    q, r = torch.linalg.qr(a)
    return q * torch.sign(torch.diagonal(r)).unsqueeze(0)


class KVLaw:
    """Per-head anisotropic Gaussian law of the synthetic KV workloads.

    ``factor[h]`` is a d x d matrix F_h with x = F_h z, z ~ N(0, I), before the
    outlier channels are scaled.
    """

    def __init__(self, num_heads: int, d: int, seed: int, device="cpu"):
        self.num_heads, self.d = num_heads, d
        g = _gen(seed, "cpu")
        lam = torch.empty(d, dtype=torch.float64)
        top = torch.tensor(KV_TOP_FRACTIONS, dtype=torch.float64)
        lam[: len(top)] = top * d
        lam[len(top):] = (1.0 - float(top.sum())) * d / (d - len(top))
        self.eigenvalues = lam
        factors, outliers = [], []
        for _ in range(num_heads):
            u = _haar(d, d, g, "cpu")
            factors.append(u * lam.sqrt().unsqueeze(0))
            outliers.append(torch.randperm(d, generator=g)[:KV_NUM_OUTLIERS])
        self.factor = torch.stack(factors).to(device)              # [H][d][d] fp64
        scale = torch.ones(num_heads, d, dtype=torch.float64)
        for h, o in enumerate(outliers):
            scale[h, o] = KV_OUTLIER_SCALE
        self.channel_scale = scale.to(device)                      # [H][d]
        self.outliers = torch.stack(outliers)

    def sample(self, head: int, n: int, g: torch.Generator, device, out_dtype=torch.bfloat16):
        z = torch.randn(n, self.d, generator=g, device=device, dtype=torch.float32)
        f = self.factor[head].to(device=device, dtype=torch.float32)
        x = (z @ f.T) * self.channel_scale[head].to(device=device, dtype=torch.float32)
        return x.to(out_dtype)

    def realised_top4_fraction(self, head: int) -> float:
        """Fraction of the trace in the 4 largest eigenvalues after the outlier scaling."""
        f = self.factor[head].cpu() * self.channel_scale[head].cpu().unsqueeze(1)
        ev = torch.linalg.eigvalsh(f @ f.T).flip(0)
        return float(ev[:4].sum() / ev.sum())


def kv_cache(batch: int, heads: int, tokens: int, d: int, seed: int, law: KVLaw,
             device="cpu", chunk: int = 1 << 20) -> torch.Tensor:
    """bf16 tensor [batch][heads][tokens][d] drawn from ``law``."""
    out = torch.empty(batch, heads, tokens, d, dtype=torch.bfloat16, device=device)
    g = _gen(seed, device)
    for b in range(batch):
        for h in range(heads):
            for t0 in range(0, tokens, chunk):
                t1 = min(tokens, t0 + chunk)
                out[b, h, t0:t1] = law.sample(h, t1 - t0, g, device)
    return out


def kv_queries(batch: int, q_heads: int, kv_heads: int, d: int, seed: int, law: KVLaw,
               device="cpu") -> torch.Tensor:
    """bf16 queries [batch][q_heads][d]; query head h follows the law of KV head h // (q_heads // kv_heads)."""
    group = q_heads // kv_heads
    g = _gen(seed, device)
    q = torch.empty(batch, q_heads, d, dtype=torch.bfloat16, device=device)
    for h in range(q_heads):
        q[:, h] = law.sample(h // group, batch, g, device)
    return q


class LowRankLaw:
    """Unit-norm vectors: half the energy isotropic, half in a rank-r subspace."""

    def __init__(self, d: int, rank: int, seed: int, device="cpu"):
        self.d, self.rank = d, rank
        g = _gen(seed, "cpu")
        self.basis = _haar(d, rank, g, "cpu").to(device=device, dtype=torch.float32)

    def sample(self, n: int, g: torch.Generator, device) -> torch.Tensor:
        iso = torch.randn(n, self.d, generator=g, device=device) / math.sqrt(2 * self.d)
        z = torch.randn(n, self.rank, generator=g, device=device) / math.sqrt(2 * self.rank)
        x = iso + z @ self.basis.to(device).T
        return x / x.norm(dim=1, keepdim=True)


def lowrank_vectors(n: int, law: LowRankLaw, seed: int, device="cpu", chunk: int = 1 << 18,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """n x d fp32 rows from ``law``, drawn in chunks so large databases fit."""
    if out is None:
        out = torch.empty(n, law.d, dtype=torch.float32, device=device)
    g = _gen(seed, device)
    for i in range(0, n, chunk):
        j = min(n, i + chunk)
        out[i:j] = law.sample(j - i, g, device)
    return out


# Seeds per workload: data = 100c+1, queries = 100c+2, rotation = 100c+3,
# sketch = 100c+4, calibration = 100c+5, with c the workload number below.
WORKLOADS = {
    1: "prod b=3, d=128, 4096 iid fp32 vectors, 16 queries",
    2: "GQA decode layer: 32 q heads / 8 kv heads, d=128, 32768 tokens, bf16",
    3: "bulk prefill encode: 32 layers x 8 kv heads x 131072 tokens, d=128, bf16",
    4: "SpectralQuant batched decode: 64 seqs x 8192 tokens, 8 kv / 32 q heads, bf16",
    5: "vector search: 1e6 x 1536 unit vectors (rank-64 half energy), 1024 queries, top-10",
}


def seed(workload: int, role: str) -> int:
    return 100 * workload + {"data": 1, "queries": 2, "rotation": 3, "sketch": 4,
                             "calibration": 5, "values": 6, "vrotation": 7}[role]


def random_codes(n: int, d: int, levels: int, m: int, seed: int):
    """Arbitrary stored codes for scoring tests: indices uniform in [0, levels),
    sign bits fair coins, n_x uniform in [0.5, 1.5) and n_r in [0.05, 0.7),
    both as fp16.  Returns (idx [n][d] int64, signs [n][m] bool or None, nx, nr)."""
    g = np.random.Generator(np.random.Philox(seed))
    idx = g.integers(0, levels, size=(n, d), dtype=np.int64)
    signs = g.integers(0, 2, size=(n, m), dtype=np.uint8).astype(bool) if m > 0 else None
    nx = g.uniform(0.5, 1.5, size=n).astype(np.float16)
    nr = g.uniform(0.05, 0.7, size=n).astype(np.float16) if m > 0 else None
    return idx, signs, nx, nr
