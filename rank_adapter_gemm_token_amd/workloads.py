"""Seeded synthetic inputs for the adapter execution unit.

This module draws inputs only: shapes, value distributions, adapter indices.
It holds none of the method's arithmetic and imports neither the HIP library
nor the oracle, so both sides can take their inputs from it.

Workloads (all shapes are 7B-decoder shaped; "a x b" reads d_in x d_out):

  tiny     one 256x256 fp32 linear, 4 adapters r=8 alpha=16, 16 tokens, idx
           uniform over {base_only, 0, 1, 2, 3}
  decode   q_proj 4096x4096 fp16, 6 adapters r=16 alpha=32, 64 tokens, idx
           uniform over the 6 adapters with 10% base_only
  sweep    4096x4096 fp16, 100 adapters r=8 alpha=16, T in {1,8,16,32,64},
           idx drawn from a finite Zipf(s=1.1) over the 100 slots
  prefill  q_proj and v_proj 4096x4096 bf16, 32 adapters per projection with
           ranks from {8,16,32,64} padded to 64, alpha = 2r, 8 sequences x 512
           tokens, one adapter per sequence (contiguous)
  stack    32 layers x {q,k,v,o 4096x4096; gate,up 4096x11008; down 11008x4096}
           bf16, 64 adapters r=16 alpha=32 on every projection, 256 tokens,
           Zipf(1.1) idx + 5% base_only
  shard    one GPU's share of the decode q_proj split eight ways: "col"
           4096x512 (output columns sharded: W and B by column, A whole),
           "row" 512x4096 (input rows sharded: W and A by row, B whole); 6
           adapters r=16 alpha=32, 64 tokens, the decode idx

Value distributions, N(0, v) with v the variance: x ~ N(0, 1); W, A ~
N(0, 1/d_in); B ~ N(0, 0.01).  Small and medium tensors are drawn in fp64
with numpy's PCG64 and rounded to the pool dtype by torch; the stack's weights
(13 GB) are drawn on the device with a seeded torch generator.  Parity never
depends on the generator: the oracle reads back the exact stored bits.
"""
from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np
import torch

BASE_ONLY = -1

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

STACK_SHAPES = [  # (name, d_in, d_out) for one decoder layer
    ("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096), ("gate_proj", 4096, 11008), ("up_proj", 4096, 11008),
    ("down_proj", 11008, 4096),
]
STACK_LAYERS = 32


@dataclass
class Adapter:
    slot: int
    tenant: int
    rank: int
    alpha: float
    A: torch.Tensor  # [rank][d_in]
    B: torch.Tensor  # [d_out][rank]


@dataclass
class Linear:
    name: str
    d_in: int
    d_out: int
    W: torch.Tensor  # [d_out][d_in], nn.Linear layout
    adapters: List[Adapter] = field(default_factory=list)


@dataclass
class Workload:
    name: str
    dtype: str          # "f32" | "f16" | "bf16"
    T: int
    S: int              # adapter slots per pool
    R: int              # pool's common (padded) rank
    idx: torch.Tensor   # [T] int32, BASE_ONLY = -1
    x: Dict[int, torch.Tensor]  # d_in -> [T][d_in]
    linears: List[Linear]
    seed: int
    notes: str = ""


def zipf_pmf(n: int, s: float) -> np.ndarray:
    """Finite Zipf law over ranks 1..n: P(k) proportional to k^-s."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def draw_idx(rng, T, n_slots, dist="uniform", base_only=0.0, s=1.1):
    """Per-token adapter slots; a token is base_only with probability base_only."""
    if dist == "uniform":
        slots = rng.integers(0, n_slots, size=T)
    elif dist == "zipf":
        slots = rng.choice(n_slots, size=T, p=zipf_pmf(n_slots, s))
    else:
        raise ValueError(dist)
    if base_only > 0.0:
        mask = rng.random(T) < base_only
        slots = np.where(mask, BASE_ONLY, slots)
    return torch.from_numpy(slots.astype(np.int32))


def normal(rng, shape, var, dtype):
    """N(0, var) drawn in fp64, rounded to dtype."""
    a = rng.standard_normal(size=shape) * np.sqrt(var)
    return torch.from_numpy(a).to(DTYPES[dtype])


def _adapters(rng, n, d_in, d_out, ranks, alphas, dtype):
    out = []
    for i in range(n):
        r = int(ranks[i])
        out.append(Adapter(slot=i, tenant=i, rank=r, alpha=float(alphas[i]),
                           A=normal(rng, (r, d_in), 1.0 / d_in, dtype),
                           B=normal(rng, (d_out, r), 0.01, dtype)))
    return out


def tiny(seed=1) -> Workload:
    rng = np.random.default_rng(seed)
    d, T, S, r = 256, 16, 4, 8
    x = normal(rng, (T, d), 1.0, "f32")
    W = normal(rng, (d, d), 1.0 / d, "f32")
    ad = _adapters(rng, S, d, d, [r] * S, [16.0] * S, "f32")
    idx = torch.from_numpy((rng.integers(0, S + 1, size=T) - 1).astype(np.int32))
    return Workload("tiny 256x256 fp32, 4 adapters r8, 16 tokens", "f32", T, S, r, idx,
                    {d: x}, [Linear("linear", d, d, W, ad)], seed)


def decode(seed=2, T=64) -> Workload:
    rng = np.random.default_rng(seed)
    d, S, r = 4096, 6, 16
    x = normal(rng, (T, d), 1.0, "f16")
    W = normal(rng, (d, d), 1.0 / d, "f16")
    ad = _adapters(rng, S, d, d, [r] * S, [32.0] * S, "f16")
    idx = draw_idx(rng, T, S, "uniform", base_only=0.10)
    return Workload("decode q_proj 4096x4096 fp16, 6 adapters r16, %d tokens" % T, "f16",
                    T, S, r, idx, {d: x}, [Linear("q_proj", d, d, W, ad)], seed)


def shard(kind, seed=2, T=64, parts=8) -> Workload:
    """The decode q_proj's per-GPU shard under eight-way tensor parallelism,
    drawn with the decode workload's distributions (W, A ~ N(0, 1/4096), the
    variance of the full 4096-wide projection)."""
    rng = np.random.default_rng(seed + 100)
    d, S, r = 4096, 6, 16
    if kind == "col":
        d_in, d_out = d, d // parts
    elif kind == "row":
        d_in, d_out = d // parts, d
    else:
        raise ValueError(kind)
    x = normal(rng, (T, d_in), 1.0, "f16")
    W = normal(rng, (d_out, d_in), 1.0 / d, "f16")
    ad = []
    for i in range(S):
        ad.append(Adapter(slot=i, tenant=i, rank=r, alpha=32.0,
                          A=normal(rng, (r, d_in), 1.0 / d, "f16"),
                          B=normal(rng, (d_out, r), 0.01, "f16")))
    idx = draw_idx(rng, T, S, "uniform", base_only=0.10)
    return Workload("shard-%s q_proj %dx%d fp16, 6 adapters r16, %d tokens" % (kind, d_in, d_out, T), "f16",
                    T, S, r, idx, {d_in: x}, [Linear("q_proj", d_in, d_out, W, ad)], seed)


SWEEP_T = (1, 8, 16, 32, 64)


def sweep(T, seed=3) -> Workload:
    """100-adapter pool; the weights depend on the seed only, idx on (seed, T)."""
    rng = np.random.default_rng(seed)
    d, S, r = 4096, 100, 8
    W = normal(rng, (d, d), 1.0 / d, "f16")
    ad = _adapters(rng, S, d, d, [r] * S, [16.0] * S, "f16")
    rng_t = np.random.default_rng([seed, T])
    x = normal(rng_t, (T, d), 1.0, "f16")
    idx = draw_idx(rng_t, T, S, "zipf", base_only=0.0)
    return Workload("sweep 4096x4096 fp16, 100 adapters r8, %d tokens" % T, "f16",
                    T, S, r, idx, {d: x}, [Linear("linear", d, d, W, ad)], seed)


def prefill(seed=4, n_seq=8, seq_len=512) -> Workload:
    rng = np.random.default_rng(seed)
    d, S, R = 4096, 32, 64
    T = n_seq * seq_len
    ranks = rng.choice(np.array([8, 16, 32, 64]), size=S)
    alphas = 2.0 * ranks
    seq_slot = rng.integers(0, S, size=n_seq)
    idx = torch.from_numpy(np.repeat(seq_slot, seq_len).astype(np.int32))
    x = normal(rng, (T, d), 1.0, "bf16")
    linears = []
    for name in ("q_proj", "v_proj"):
        W = normal(rng, (d, d), 1.0 / d, "bf16")
        ad = _adapters(rng, S, d, d, ranks, alphas, "bf16")
        linears.append(Linear(name, d, d, W, ad))
    return Workload("prefill q_proj+v_proj 4096x4096 bf16, 32 adapters r{8..64} pad 64, "
                    "8x512 tokens", "bf16", T, S, R, idx, {d: x}, linears, seed,
                    notes="seq_slot=%s ranks=%s" % (seq_slot.tolist(), ranks.tolist()))


def stack_idx(seed=5, T=256, S=64):
    rng = np.random.default_rng(seed)
    return draw_idx(rng, T, S, "zipf", base_only=0.05)


def stack_x(d_in, seed=5, T=256, device="cpu"):
    rng = np.random.default_rng([seed, d_in])
    return normal(rng, (T, d_in), 1.0, "bf16").to(device)


def stack_linear(layer, proj, device, seed=5, S=64, r=16) -> Linear:
    """One linear of the 7B stack, drawn on `device` with a seeded torch generator.

    Three draws per linear (W, then every adapter's A at once, then every B):
    a few large dispatches rather than one pair per adapter, which keeps the
    set-up of the 224-linear stack to a few hundred device dispatches."""
    name, d_in, d_out = STACK_SHAPES[proj]
    g = torch.Generator(device=device)
    g.manual_seed(1000 * seed + 8 * layer + proj)

    def randn(shape, var):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return t.mul_(float(np.sqrt(var))).to(torch.bfloat16)

    W = randn((d_out, d_in), 1.0 / d_in)
    A_all = randn((S, r, d_in), 1.0 / d_in)
    B_all = randn((S, d_out, r), 0.01)
    ad = [Adapter(slot=i, tenant=i, rank=r, alpha=2.0 * r, A=A_all[i], B=B_all[i]) for i in range(S)]
    return Linear("layer%d.%s" % (layer, name), d_in, d_out, W, ad)


def stack(seed=5, T=256, device="cuda", layers=STACK_LAYERS) -> Workload:
    S, R = 64, 16
    idx = stack_idx(seed, T, S)
    xs = {4096: stack_x(4096, seed, T, device), 11008: stack_x(11008, seed, T, device)}
    linears = [stack_linear(l, p, device, seed, S, R)
               for l in range(layers) for p in range(len(STACK_SHAPES))]
    return Workload("stack 7B decoder linears bf16 (32 layers x 7), 64 adapters r16, "
                    "256 tokens", "bf16", T, S, R, idx, xs, linears, seed)
