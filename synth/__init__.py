"""Seeded synthetic inputs for the MoE grouped-GEMM path.

This module is shared by the tests, the benchmark and the smoke check. It
draws router outputs, activations and expert weights with fixed seeds and
holds none of the method's arithmetic: no FP8/INT4 quantisation, no
routing/packing, no GEMM and no combine.  Every value it returns is a plain
random draw (rounded to bf16 where the workload says bf16), a top-k of random
router logits, or a softmax of random router logits.

Workloads (shapes as the MoE layers of DeepSeek-V3 and Qwen3-235B; the pages
give the layouts and number formats, the sizes below are the ones measured):

  tiny          T=64,   E=4,   top-2, K=256,  N=256,  contiguous (128-row aligned), FP8
  dsv3_prefill  T=4096, E=256, top-8, K=7168, N=4096, contiguous (128-row aligned), FP8
  dsv3_decode   T=128,  E=256, top-8, K=7168, N=4096, masked (64 rows per expert), FP8
  qwen3_skewed  T=8192, E=128, top-8 Zipf(1.1), up K=4096 N=3072, down K=1536 N=4096, FP8
  int4_decode   T=16,   E=128, top-8, K=4096, N=1536, masked (16 rows per expert), INT4

Recipes:
  * uniform routing: router logits ~ N(0,1) of shape [T, E]; topk_ids are the
    k largest logits per token, in descending order (distinct experts).
  * Zipf routing: expert popularity p_e proportional to (e+1)^-s; k distinct
    experts per token drawn without replacement by Gumbel-top-k on log p_e.
    An optional permutation maps popularity rank to expert id.
  * topk_weights: softmax of k fresh N(0,1) draws per token (rows sum to 1).
  * activations: N(0,1) drawn in fp32, rounded to bf16 (RNE).
  * expert weights: N(0, 0.02) drawn in fp32 per expert, rounded to bf16.

Seeds are derived from (workload index, stream id, sub-index) so that one
expert's weights can be regenerated alone.  On the CPU the draws come from
torch's CPU generator; on a GPU from torch's device generator (identical
recipe, different stream of numbers).  Tests that compare against the oracle
either generate on the CPU and copy to the device, or copy the sampled rows
of device-generated inputs back to the host.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

__all__ = [
    "MoeConfig",
    "CONFIGS",
    "config_by_name",
    "seed_for",
    "route_inputs",
    "activations",
    "expert_weights",
    "STREAM_ROUTE",
    "STREAM_ROUTE_WEIGHTS",
    "STREAM_ACT",
    "STREAM_ACT_DOWN",
    "STREAM_WEIGHTS",
    "STREAM_WEIGHTS_DOWN",
]

STREAM_ROUTE = 0
STREAM_ROUTE_WEIGHTS = 1
STREAM_ACT = 2
STREAM_ACT_DOWN = 3
STREAM_WEIGHTS = 100
STREAM_WEIGHTS_DOWN = 200


@dataclass(frozen=True)
class MoeConfig:
    index: int
    name: str
    T: int
    E: int
    topk: int
    K: int
    N: int
    routing: str = "uniform"  # "uniform" | "zipf"
    zipf_s: float = 1.1
    layout: str = "contiguous"  # "contiguous" | "masked"
    align: int = 128
    max_m: int = 0
    weights: str = "fp8"  # "fp8" | "int4"
    w_std: float = 0.02
    K_down: int = 0
    N_down: int = 0
    weight_seed_index: int = -1  # share another workload's expert weights
    notes: str = field(default="", compare=False)

    @property
    def R(self) -> int:
        return self.T * self.topk

    @property
    def wseed(self) -> int:
        return self.index if self.weight_seed_index < 0 else self.weight_seed_index


CONFIGS = [
    MoeConfig(0, "tiny", T=64, E=4, topk=2, K=256, N=256),
    MoeConfig(1, "dsv3_prefill", T=4096, E=256, topk=8, K=7168, N=4096),
    MoeConfig(2, "dsv3_decode", T=128, E=256, topk=8, K=7168, N=4096,
              layout="masked", max_m=64, weight_seed_index=1),
    MoeConfig(3, "qwen3_skewed", T=8192, E=128, topk=8, K=4096, N=3072,
              routing="zipf", zipf_s=1.1, K_down=1536, N_down=4096),
    MoeConfig(4, "int4_decode", T=16, E=128, topk=8, K=4096, N=1536,
              layout="masked", max_m=16, weights="int4"),
]


def config_by_name(name: str) -> MoeConfig:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def seed_for(cfg_index: int, stream: int, sub: int = 0, seed: int = 0) -> int:
    """Deterministic 63-bit seed for (workload, stream, sub-index, user seed)."""
    x = (cfg_index + 1) * 0x9E3779B97F4A7C15 + (stream + 1) * 0xBF58476D1CE4E5B9
    x += (sub + 1) * 0x94D049BB133111EB + (seed + 1) * 0x2545F4914F6CDD1D
    x &= (1 << 64) - 1
    x ^= x >> 31
    return x & ((1 << 63) - 1)


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def route_inputs(cfg: MoeConfig, seed: int = 0, T: int | None = None,
                 perm: torch.Tensor | None = None):
    """Router outputs (topk_ids int32 [T,k], topk_weights float32 [T,k]) on the CPU."""
    T = cfg.T if T is None else T
    E, k = cfg.E, cfg.topk
    g = _gen("cpu", seed_for(cfg.index, STREAM_ROUTE, 0, seed))
    if cfg.routing == "uniform":
        logits = torch.randn(T, E, generator=g, dtype=torch.float32)
    elif cfg.routing == "zipf":
        logp = -cfg.zipf_s * torch.log(torch.arange(1, E + 1, dtype=torch.float64))
        u = torch.rand(T, E, generator=g, dtype=torch.float64).clamp_(min=1e-300)
        gumbel = -torch.log(-torch.log(u))
        logits = logp[None, :] + gumbel
    else:
        raise ValueError(cfg.routing)
    ids = torch.topk(logits, k, dim=1, largest=True, sorted=True).indices
    if perm is not None:
        ids = perm[ids]
    g2 = _gen("cpu", seed_for(cfg.index, STREAM_ROUTE_WEIGHTS, 0, seed))
    w = torch.softmax(torch.randn(T, k, generator=g2, dtype=torch.float32), dim=1)
    return ids.to(torch.int32).contiguous(), w.contiguous()


def activations(cfg: MoeConfig, rows: int, K: int, stream: int = STREAM_ACT,
                device="cpu", seed: int = 0) -> torch.Tensor:
    """bf16 [rows, K] with values N(0,1) drawn in fp32 and rounded to bf16."""
    g = _gen(device, seed_for(cfg.index, stream, 0, seed))
    x = torch.randn(rows, K, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def expert_weights(cfg: MoeConfig, N: int, K: int, experts=None,
                   stream: int = STREAM_WEIGHTS, device="cpu", seed: int = 0,
                   E: int | None = None) -> torch.Tensor:
    """bf16 [len(experts), N, K] with values N(0, w_std), one seeded draw per expert.

    ``experts`` selects which experts to produce (default: all E); expert e is
    always drawn from the same seed, so a subset can be regenerated alone.
    """
    E = cfg.E if E is None else E
    experts = list(range(E)) if experts is None else list(experts)
    out = torch.empty(len(experts), N, K, dtype=torch.bfloat16, device=device)
    for i, e in enumerate(experts):
        g = _gen(device, seed_for(cfg.wseed, stream, e, seed))
        w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32)
        out[i] = (w * cfg.w_std).to(torch.bfloat16)
    return out


def zipf_perm(cfg: MoeConfig, seed: int = 0) -> torch.Tensor:
    """A seeded permutation of expert ids (popularity rank -> expert id)."""
    g = _gen("cpu", seed_for(cfg.index, 7, 0, seed))
    return torch.randperm(cfg.E, generator=g)


def bits_u16(t: torch.Tensor):
    """The uint16 bit patterns of a bf16/fp16 tensor as a host numpy array."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _expected_rows(cfg: MoeConfig) -> float:
    return cfg.R / cfg.E if cfg.E else 0.0


def describe(cfg: MoeConfig) -> str:
    return (f"{cfg.name}: T={cfg.T} E={cfg.E} top-{cfg.topk} K={cfg.K} N={cfg.N} "
            f"{cfg.layout} {cfg.weights} (~{_expected_rows(cfg):.1f} rows/expert)")

