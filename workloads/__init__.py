"""Seeded synthetic inputs for the KDA training recurrence.

This module only draws random numbers and lays them out in the tensor
contract of the FlashInfer training API (page "flashinfer.kda_training.
recurrent_kda_training_forward", parameter list): BF16 token tensors
[B, T, H, 128], BF16 raw beta logits [B, T, Hv], FP32 A_log [Hv], FP32
dt_bias [Hv, 128] and an FP32 value-first initial state [N, Hv, 128, 128].
It holds none of the method's arithmetic, so both the oracle and the GPU
path can consume the same draws.

The five named workloads are the ones the library is measured on:

    tiny      fixed  B=1  T=64    Hqk=Hv=2
    fixed     fixed  B=2  T=2048  Hqk=Hv=16   (zero initial state)
    grouped   fixed  B=4  T=4096  Hqk=8  Hv=32
    packed    packed 8 sequences x 1024 tokens, Hqk=Hv=96
    mixed     packed 32 sequences, lengths ~U[1,4096], Hqk=16, Hv=64

Draw order (CPU torch.Generator seeded with the workload's seed):
lengths (mixed only), q, k, v, g (randn, cast to BF16), beta logits (randn,
BF16), A_log = 2*rand, dt_bias = 0.1*randn, initial_state = 0.01*randn (or
zeros), then the loss adjoints do (randn, BF16) and dfinal_state
(0.01*randn).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

DIM = 128


@dataclass
class Problem:
    """Shape description of one call. `lengths` lists the semantic sequences."""
    lengths: list
    Hqk: int
    Hv: int
    packed: bool
    zero_state: bool = False
    name: str = "custom"

    def __post_init__(self):
        if not self.lengths or min(self.lengths) < 1:
            raise ValueError("every sequence needs at least one token")
        if not self.packed and len(set(self.lengths)) != 1:
            raise ValueError("the fixed layout has one length T for every sequence")

    @property
    def N(self) -> int:
        return len(self.lengths)

    @property
    def B(self) -> int:
        return 1 if self.packed else len(self.lengths)

    @property
    def T(self) -> int:
        return sum(self.lengths) if self.packed else self.lengths[0]

    @property
    def token_heads(self) -> int:
        return sum(self.lengths) * self.Hv

    def cu_seqlens(self) -> Optional[torch.Tensor]:
        if not self.packed:
            return None
        cu = [0]
        for L in self.lengths:
            cu.append(cu[-1] + int(L))
        return torch.tensor(cu, dtype=torch.int64)


@dataclass
class Inputs:
    problem: Problem
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    initial_state: torch.Tensor
    cu_seqlens: Optional[torch.Tensor]
    do: Optional[torch.Tensor] = None
    dfinal_state: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)

    def to(self, device) -> "Inputs":
        def mv(t):
            return None if t is None else t.to(device)
        return Inputs(self.problem, mv(self.q), mv(self.k), mv(self.v), mv(self.g),
                      mv(self.beta), mv(self.A_log), mv(self.dt_bias),
                      mv(self.initial_state), mv(self.cu_seqlens), mv(self.do),
                      mv(self.dfinal_state), dict(self.extra))


def _randn_bf16(gen, shape):
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def make_inputs(problem: Problem, seed: int, with_adjoints: bool = True) -> Inputs:
    """Draw every tensor of one call from a CPU generator seeded with `seed`."""
    return _make_from_gen(problem, torch.Generator().manual_seed(seed), with_adjoints)


def mixed_lengths(seed: int, count: int = 32, max_len: int = 4096) -> list:
    """Lengths ~U[1, max_len] drawn first from the workload's generator."""
    gen = torch.Generator().manual_seed(seed)
    return [int(x) for x in torch.randint(1, max_len + 1, (count,), generator=gen)]


# Named workloads: (problem, seed). The seed of workload i is i.
def workload(name: str) -> tuple:
    if name == "tiny":
        return Problem([64], 2, 2, packed=False, name=name), 0
    if name == "fixed":
        return Problem([2048] * 2, 16, 16, packed=False, zero_state=True, name=name), 1
    if name == "grouped":
        return Problem([4096] * 4, 8, 32, packed=False, name=name), 2
    if name == "packed":
        return Problem([1024] * 8, 96, 96, packed=True, name=name), 3
    if name == "mixed":
        return Problem(mixed_lengths(4), 16, 64, packed=True, name=name), 4
    raise KeyError(name)


WORKLOADS = ("tiny", "fixed", "grouped", "packed", "mixed")


def make_workload(name: str, with_adjoints: bool = True) -> Inputs:
    """The named workload's inputs. For `mixed`, the generator first draws the
    lengths and then continues with the tensors, as one stream."""
    problem, seed = workload(name)
    if name != "mixed":
        return make_inputs(problem, seed, with_adjoints)
    # one generator stream: lengths first, then the tensors
    gen = torch.Generator().manual_seed(seed)
    _ = torch.randint(1, 4097, (32,), generator=gen)
    return _make_from_gen(problem, gen, with_adjoints)


def _make_from_gen(problem: Problem, gen, with_adjoints: bool) -> Inputs:
    B, T, Hqk, Hv, N = problem.B, problem.T, problem.Hqk, problem.Hv, problem.N
    q = _randn_bf16(gen, (B, T, Hqk, DIM))
    k = _randn_bf16(gen, (B, T, Hqk, DIM))
    v = _randn_bf16(gen, (B, T, Hv, DIM))
    g = _randn_bf16(gen, (B, T, Hv, DIM))
    beta = _randn_bf16(gen, (B, T, Hv))
    A_log = 2.0 * torch.rand((Hv,), generator=gen, dtype=torch.float32)
    dt_bias = 0.1 * torch.randn((Hv, DIM), generator=gen, dtype=torch.float32)
    if problem.zero_state:
        s0 = torch.zeros((N, Hv, DIM, DIM), dtype=torch.float32)
    else:
        s0 = 0.01 * torch.randn((N, Hv, DIM, DIM), generator=gen, dtype=torch.float32)
    do = dfs = None
    if with_adjoints:
        do = _randn_bf16(gen, (B, T, Hv, DIM))
        dfs = 0.01 * torch.randn((N, Hv, DIM, DIM), generator=gen, dtype=torch.float32)
    return Inputs(problem, q, k, v, g, beta, A_log, dt_bias, s0, problem.cu_seqlens(), do, dfs)


def make_inputs_on_device(problem: Problem, seed: int, device, with_adjoints: bool = True) -> Inputs:
    """The same recipe drawn by a generator on `device` (fast for large
    shapes; the values differ from the CPU draws of the same seed, the
    distributions do not).  Used for timing, and by the maximum-size parity
    test, which copies the sampled tasks' values back for the oracle."""
    gen = torch.Generator(device=device).manual_seed(seed)
    B, T, Hqk, Hv, N = problem.B, problem.T, problem.Hqk, problem.Hv, problem.N

    def rn(shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    q = rn((B, T, Hqk, DIM)).to(torch.bfloat16)
    k = rn((B, T, Hqk, DIM)).to(torch.bfloat16)
    v = rn((B, T, Hv, DIM)).to(torch.bfloat16)
    g = rn((B, T, Hv, DIM)).to(torch.bfloat16)
    beta = rn((B, T, Hv)).to(torch.bfloat16)
    A_log = 2.0 * torch.rand((Hv,), generator=gen, device=device, dtype=torch.float32)
    dt_bias = 0.1 * rn((Hv, DIM))
    s0 = torch.zeros((N, Hv, DIM, DIM), dtype=torch.float32, device=device) if problem.zero_state \
        else 0.01 * rn((N, Hv, DIM, DIM))
    do = dfs = None
    if with_adjoints:
        do = rn((B, T, Hv, DIM)).to(torch.bfloat16)
        dfs = 0.01 * rn((N, Hv, DIM, DIM))
    cu = problem.cu_seqlens()
    return Inputs(problem, q, k, v, g, beta, A_log, dt_bias, s0,
                  None if cu is None else cu.to(device), do, dfs, {"cu_seqlens_cpu": cu})


def sequence_slices(problem: Problem):
    """(n, b, t0, L): sequence n lives in batch row b at tokens [t0, t0+L)."""
    out = []
    if problem.packed:
        t0 = 0
        for n, L in enumerate(problem.lengths):
            out.append((n, 0, t0, int(L)))
            t0 += int(L)
    else:
        for n, L in enumerate(problem.lengths):
            out.append((n, n, 0, int(L)))
    return out


@dataclass
class InferInputs:
    """One inference call (page "flashinfer.kda.recurrent_kda"): token tensors
    as in the training contract, a BF16 state pool [P, Hv, 128, 128] and the
    pool slot of every sequence."""
    problem: Problem
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    pool: torch.Tensor
    indices: torch.Tensor
    cu_seqlens: Optional[torch.Tensor]


def make_infer_inputs(problem: Problem, seed: int, pool_slots: int, log_gate_min: float = -5.0,
                      beta_logits: bool = False, qk_std: float = 1.0) -> InferInputs:
    """Draw order (CPU generator seeded with `seed`): q, k (qk_std * randn,
    BF16), v (randn, BF16), g, beta, A_log = 2*rand, dt_bias = 0.1*randn,
    pool = 0.1*randn (BF16), indices = the first N of a permutation of the
    pool's slots.  g is a raw gate input (randn) when log_gate_min is None,
    else a log-space decay uniform in (log_gate_min, 0); beta is a logit
    (randn) or a rate uniform in (0, 1).  qk_std near 1/sqrt(128) gives
    near-unit keys for calls that skip the L2 norm."""
    gen = torch.Generator().manual_seed(seed)
    B, T, Hqk, Hv, N = problem.B, problem.T, problem.Hqk, problem.Hv, problem.N
    q = (qk_std * torch.randn((B, T, Hqk, DIM), generator=gen)).to(torch.bfloat16)
    k = (qk_std * torch.randn((B, T, Hqk, DIM), generator=gen)).to(torch.bfloat16)
    v = _randn_bf16(gen, (B, T, Hv, DIM))
    if log_gate_min is None:
        g = _randn_bf16(gen, (B, T, Hv, DIM))
    else:
        g = (log_gate_min * torch.rand((B, T, Hv, DIM), generator=gen)).to(torch.bfloat16)
    if beta_logits:
        beta = _randn_bf16(gen, (B, T, Hv))
    else:
        beta = torch.rand((B, T, Hv), generator=gen).to(torch.bfloat16)
    A_log = 2.0 * torch.rand((Hv,), generator=gen, dtype=torch.float32)
    dt_bias = 0.1 * torch.randn((Hv, DIM), generator=gen, dtype=torch.float32)
    pool = (0.1 * torch.randn((pool_slots, Hv, DIM, DIM), generator=gen)).to(torch.bfloat16)
    indices = torch.randperm(pool_slots, generator=gen)[:N].to(torch.int32)
    return InferInputs(problem, q, k, v, g, beta, A_log, dt_bias, pool, indices,
                       problem.cu_seqlens())
