"""Seeded synthetic workloads for the KDA forward pass.

Random-number recipes and shapes only: this module contains none of the
method's arithmetic, and it is the one piece of code that both the GPU tests
and the oracle-side tests use, so both consume bit-identical inputs.

Recipe: a CPU torch.Generator seeded per workload; tensors are drawn in the
order lengths (ragged batches only), q, k, v, g_raw, beta_raw, initial_state,
as fp32 standard normals that are shifted/scaled and then rounded to the I/O
dtype (round-to-nearest-even for bf16).

Named workloads (T = tokens, H = heads, head dim 128, lower_bound = -5):
  c1  one sequence, T=64, H=1, fp32 I/O, all N(0,1), zero initial state, seed 0
  c2  one sequence, T=4096, H=16, bf16, all N(0,1), zero initial state, seed 1
  c3  8 packed sequences x 8192 tokens (cu_seqlens), H=32, bf16, all N(0,1),
      initial state N(0, 0.02^2) per (sequence, head), seed 2
  c4  one sequence, T=131072, H=32, bf16, g_raw ~ N(-1,1), zero initial state, seed 3
  c5  64 packed sequences with lengths uniform in [256, 4096], H=32, bf16,
      g_raw ~ N(0,1), beta_raw ~ N(1,1), initial state N(0, 0.02^2), seed 4
  d1  one decode step: 256 packed sequences x 1 token, H=32, bf16, all N(0,1),
      initial state N(0, 0.02^2), seed 5
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

HEAD_DIM = 128


@dataclass
class Workload:
    name: str
    q: torch.Tensor          # [T_tot, H, 128] (packed) -- see `batch`
    k: torch.Tensor
    v: torch.Tensor
    g_raw: torch.Tensor
    beta_raw: torch.Tensor   # [T_tot, H]
    seq_lens: list            # lengths of the N sequences
    packed: bool              # True: pass cu_seqlens; False: batch rows of equal length
    initial_state: torch.Tensor | None  # [N, H, 128, 128] fp32 or None
    lower_bound: float = -5.0
    meta: dict = field(default_factory=dict)

    @property
    def T_tot(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def N(self) -> int:
        return len(self.seq_lens)

    def offsets(self) -> list:
        o = [0]
        for L in self.seq_lens:
            o.append(o[-1] + int(L))
        return o

    def cu_seqlens(self) -> torch.Tensor:
        return torch.tensor(self.offsets(), dtype=torch.int32)


def _draw(gen, shape, mean=0.0, std=1.0, dtype=torch.bfloat16):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(dtype)


def make(seq_lens, H, *, seed, dtype=torch.bfloat16, packed=True, g_mean=0.0, beta_mean=0.0,
         init_std=0.0, lower_bound=-5.0, name="custom", lens_drawn=None, scalar_gate=False) -> Workload:
    """Generic seeded workload. seq_lens: list of sequence lengths. scalar_gate:
    g_raw is drawn as [T, H] (one gate per token and head) instead of [T, H, 128]."""
    gen = torch.Generator().manual_seed(int(seed))
    if lens_drawn is not None:  # ragged lengths are the first draw
        lo, hi, count = lens_drawn
        seq_lens = torch.randint(lo, hi + 1, (count,), generator=gen).tolist()
    T = int(sum(seq_lens))
    shape = (T, H, HEAD_DIM)
    q = _draw(gen, shape, dtype=dtype)
    k = _draw(gen, shape, dtype=dtype)
    v = _draw(gen, shape, dtype=dtype)
    g = _draw(gen, (T, H) if scalar_gate else shape, mean=g_mean, dtype=dtype)
    b = _draw(gen, (T, H), mean=beta_mean, dtype=dtype)
    s0 = None
    if init_std > 0:
        s0 = _draw(gen, (len(seq_lens), H, HEAD_DIM, HEAD_DIM), std=init_std, dtype=torch.float32)
    return Workload(name, q, k, v, g, b, list(seq_lens), packed, s0, lower_bound,
                    dict(seed=seed, dtype=str(dtype), g_mean=g_mean, beta_mean=beta_mean, init_std=init_std,
                         scalar_gate=scalar_gate))


def c1() -> Workload:
    return make([64], 1, seed=0, dtype=torch.float32, packed=False, name="c1")


def c2() -> Workload:
    return make([4096], 16, seed=1, packed=False, name="c2")


def c3() -> Workload:
    return make([8192] * 8, 32, seed=2, packed=True, init_std=0.02, name="c3")


def c4() -> Workload:
    return make([131072], 32, seed=3, packed=False, g_mean=-1.0, name="c4")


def c5() -> Workload:
    return make(None, 32, seed=4, packed=True, beta_mean=1.0, init_std=0.02, name="c5",
                lens_drawn=(256, 4096, 64))


def d1() -> Workload:
    return make([1] * 256, 32, seed=5, packed=True, init_std=0.02, name="d1")


CONFIGS = {"c1": c1, "c2": c2, "c3": c3, "c4": c4, "c5": c5, "d1": d1}

DESCRIPTIONS = {
    "c1": "single sequence T=64 H=1 D=128 fp32 I/O, zero initial state",
    "c2": "single sequence T=4096 H=16 D=128 bf16, zero initial state",
    "c3": "packed varlen 8 x 8192 tokens H=32 D=128 bf16, initial state N(0,0.02^2)",
    "c4": "long context T=131072 H=32 D=128 bf16, g_raw ~ N(-1,1), zero initial state",
    "c5": "ragged varlen 64 sequences, lengths U[256,4096], H=32 D=128 bf16, beta_raw ~ N(1,1), "
          "initial state N(0,0.02^2)",
    "d1": "decode step: 256 sequences x 1 token, H=32 D=128 bf16, initial state N(0,0.02^2)",
}
