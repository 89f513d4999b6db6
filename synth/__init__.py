"""Seeded synthetic decode workloads ("cone geometry") for the MagicPIG path.

This module only draws inputs: keys, values and queries.  It holds none of the
estimator's arithmetic, and both the HIP path and the fp64 oracle take the
tensors it returns unchanged.

The geometry follows the observations on the page "MagicPIG: LSH Sampling for
Efficient LLM Generation" (background section, geometry observations 1-3) and
the page "MagicPIG: don't pick the tallest" (section 4): apart from the
first-token sink, keys of a head sit in a narrow cone whose mean points away
from both the sink key and the queries.  Per KV head a random unit direction m
is drawn and

    k_i = -2 m + N(0, I)/sqrt(d)      (ordinary keys)
    k_0 =  6 m                        (sink key, position 0)
    q   =  2 m + N(0, I)/sqrt(d)      (each query head of the group)
    v_i ~  N(0, I)

With ``tail_frac`` > 0 that fraction of the non-sink positions of each KV head,
chosen uniformly without replacement, are redrawn near +m:
k = +m + N(0, I)/sqrt(d); this makes a long tail of mid-weight tokens.

Every draw comes from one ``torch.Generator`` per sequence, seeded with that
sequence's seed, in the fixed order m, key noise, values, query noise, tail
positions.  Values are drawn in fp32 and then rounded to the storage dtype
(bf16 rounding is round-to-nearest-even); queries stay fp32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Config", "CONFIGS", "cone_inputs", "config_inputs"]


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H_q: int
    H_kv: int
    n: int
    d: int
    dtype: torch.dtype          # K/V storage dtype
    K: int
    L: int
    n_sink: int
    n_local: int
    seed: int                   # input seed of sequence 0, also the hyperplane seed
    tail_frac: float = 0.0
    per_sequence_seed: bool = False
    layers: int = 1
    l_sweep: tuple = field(default_factory=tuple)

    def seeds(self, layer: int = 0) -> list[int]:
        base = self.seed + layer
        if self.per_sequence_seed:
            return [base + 100 * b for b in range(self.B)]
        return [base] * self.B

    def hyperplane_seed(self, layer: int = 0) -> int:
        return self.seed + layer


# The five workloads of the decode benchmark.  Seeds: 1000*c + layer (c = config
# number); the tiny case uses seed 0.
CONFIGS = {
    "tiny": Config("tiny", B=1, H_q=1, H_kv=1, n=1024, d=128, dtype=torch.float32,
                   K=4, L=16, n_sink=1, n_local=16, seed=0),
    "llama8b_16k": Config("llama8b_16k", B=1, H_q=32, H_kv=8, n=16384, d=128,
                          dtype=torch.bfloat16, K=10, L=150, n_sink=4, n_local=64,
                          seed=1000),
    "llama8b_96k": Config("llama8b_96k", B=1, H_q=32, H_kv=8, n=98304, d=128,
                          dtype=torch.bfloat16, K=10, L=150, n_sink=4, n_local=64,
                          seed=2000, layers=32),
    "batch16_32k": Config("batch16_32k", B=16, H_q=32, H_kv=8, n=32768, d=128,
                          dtype=torch.bfloat16, K=10, L=150, n_sink=4, n_local=64,
                          seed=3000, tail_frac=0.10, per_sequence_seed=True),
    "llama70b_256k": Config("llama70b_256k", B=1, H_q=64, H_kv=8, n=262144, d=128,
                            dtype=torch.bfloat16, K=9, L=120, n_sink=4, n_local=64,
                            seed=4000, l_sweep=(60, 120, 240)),
}


def _one_sequence(gen, H_q, H_kv, n, d, tail_frac, device):
    G = H_q // H_kv
    inv = 1.0 / math.sqrt(d)
    m = torch.randn(H_kv, d, generator=gen, device=device, dtype=torch.float32)
    m = m / m.norm(dim=-1, keepdim=True)
    k = torch.randn(H_kv, n, d, generator=gen, device=device, dtype=torch.float32)
    k.mul_(inv).add_(-2.0 * m[:, None, :])
    k[:, 0, :] = 6.0 * m
    v = torch.randn(H_kv, n, d, generator=gen, device=device, dtype=torch.float32)
    qn = torch.randn(H_q, d, generator=gen, device=device, dtype=torch.float32)
    q = qn * inv + 2.0 * m.repeat_interleave(G, dim=0)
    if tail_frac > 0.0 and n > 1:
        n_tail = int(round(tail_frac * (n - 1)))
        for h in range(H_kv):
            pos = torch.randperm(n - 1, generator=gen, device=device)[:n_tail] + 1
            noise = torch.randn(n_tail, d, generator=gen, device=device, dtype=torch.float32)
            k[h, pos, :] = m[h][None, :] + noise * inv
    return k, v, q, m


def cone_inputs(*, B, H_q, H_kv, n, d, dtype, seeds, tail_frac=0.0, device="cpu"):
    """Return dict(k=[B][H_kv][n][d] dtype, v=same, q=[B][H_q][d] fp32, m=[B][H_kv][d])."""
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    if len(seeds) != B:
        raise ValueError("one seed per sequence")
    dev = torch.device(device)
    ks, vs, qs, ms = [], [], [], []
    for b in range(B):
        gen = torch.Generator(device=dev)
        gen.manual_seed(int(seeds[b]))
        k, v, q, m = _one_sequence(gen, H_q, H_kv, n, d, tail_frac, dev)
        ks.append(k.to(dtype))
        vs.append(v.to(dtype))
        qs.append(q)
        ms.append(m)
        del k, v
    return dict(k=torch.stack(ks), v=torch.stack(vs), q=torch.stack(qs), m=torch.stack(ms))


def config_inputs(cfg: Config, layer: int = 0, device="cpu", n=None, B=None):
    """Inputs of one layer of a named workload (optionally shrunk in n or B)."""
    nn_ = cfg.n if n is None else n
    BB = cfg.B if B is None else B
    seeds = cfg.seeds(layer)[:BB] if B is not None else cfg.seeds(layer)
    if len(seeds) < BB:
        seeds = [cfg.seed + layer + 100 * b for b in range(BB)]
    return cone_inputs(B=BB, H_q=cfg.H_q, H_kv=cfg.H_kv, n=nn_, d=cfg.d, dtype=cfg.dtype,
                       seeds=seeds, tail_frac=cfg.tail_frac, device=device)
