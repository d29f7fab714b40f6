"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds none of the verification arithmetic: it only draws logits,
draft tokens, Markov-head factors and confidence estimates, and serves both
the GPU path and the CPU oracle with identical tensors.  Real models, suites
and traffic are not available; these inputs stand in for them.

Five workloads, named by what they are (sizes can be shrunk for tests,
keeping the recipe):

  tiny       B=1,   gamma=4, V=1000,    fp32, T=1.0: target ~ N(0, 3^2) with
             one random token per row boosted by +8; draft = target + N(0, 1).
  batched    B=32,  gamma=5, V=151936,  bf16, T=0.7: target ~ N(0, 3^2) with
             1-3 random tokens per row boosted by U(6, 10); draft = target +
             N(0, 1.5^2), rounded to bf16 after the noise is added.
  headline   B=256, gamma=7, V=129280,  bf16, T=1.0: target ~ N(0, 3^2) plus a
             Zipf(1.1) bias -1.1 ln(rank), ranks a seeded random permutation
             per row; draft = target + N(0, 1).
  markov     B=128, gamma=8, V=129280,  bf16, T=1.0, R=256: backbone logits
             ~ N(0, 3^2); U, W ~ N(0, 0.02^2); anchor tokens uniform; target
             rows 1..8 = backbone + N(0, 1), row 9 ~ N(0, 3^2).
  block      B=512, gamma=8, V=129280,  bf16, T=1.0: logits as the headline
             workload's; confidences: per-request mean mu_b ~ U(0.35, 0.95),
             decaying 3% per position, plus N(0, 0.05^2), clipped to [0, 1].

Tree verification: B=64 requests, a tree of 4 branches of 5 nodes each
(the root's 4 children start 4 chains; N = 20 nodes, depth 5, 17 nodes with
children), V=129280, bf16, T=1.0.  Target rows as the headline's (one per node and
the root); the draft row of a node with children = its target row + N(0, 1);
each child's token is drawn from softmax(draft row of its parent / T) with its
own Gumbel noise, so siblings are independent draws.

RNN head (a variant of the markov workload): its backbone logits, U, W and
anchors, plus a recurrent matrix A [R, R] ~ N(0, (0.9 / sqrt(R))^2) in bf16
(spectral radius about 0.9, so the state neither dies nor saturates).

Temperature-scaled confidences (a variant of the block workload): per-position temperatures
T_i = 1 + 0.15 (i - 1), later positions hotter, and an over-confident head
whose raw log-odds are T_i times the log-odds of the block workload's confidences
(clipped to [1e-6, 1 - 1e-6] first), so that calibrated estimates land back
on them.

Draft tokens are drawn from softmax(q / T) of the stored (rounded) draft
logits with the Gumbel-max trick, from a generator seeded 0.  Logit noise uses
a generator with the workload's own seed (below).  Generation runs on the requested
device (torch generators are per device, so CPU and GPU draws differ; a test
hands the same tensors to both sides).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

# seed: the logit noise generator's seed; conf_seed: the block workload's
# confidence draws
WORKLOADS = {
    "tiny": dict(B=1, gamma=4, V=1000, dtype=torch.float32, T=1.0, seed=1001),
    "batched": dict(B=32, gamma=5, V=151936, dtype=torch.bfloat16, T=0.7, seed=1002),
    "headline": dict(B=256, gamma=7, V=129280, dtype=torch.bfloat16, T=1.0, seed=1003),
    "markov": dict(B=128, gamma=8, V=129280, dtype=torch.bfloat16, T=1.0, R=256, seed=1004),
    "block": dict(B=512, gamma=8, V=129280, dtype=torch.bfloat16, T=1.0, seed=1005, conf_seed=2005),
}

VERIFY_SEED = 1   # Philox seed of the verification uniforms
DRAFT_SEED = 0    # seed of the draft-token draws


@dataclass
class VerifyInputs:
    workload: str
    B: int
    gamma: int
    V: int
    T: float
    p: torch.Tensor            # [B, gamma+1, V]
    q: torch.Tensor            # [B, gamma, V]
    draft: torch.Tensor        # [B, gamma] int32
    conf: Optional[torch.Tensor] = None   # [B, gamma] fp32 (block workload)
    extra: dict = field(default_factory=dict)


@dataclass
class MarkovInputs:
    B: int
    gamma: int
    V: int
    R: int
    T: float
    base: torch.Tensor         # [B, gamma, V] bf16
    U: torch.Tensor            # [V, R] bf16
    Wt: torch.Tensor           # [V, R] bf16: the transition matrix W [R, V], stored vocabulary-major
    x0: torch.Tensor           # [B] int32
    p: torch.Tensor            # [B, gamma+1, V] bf16 target logits

    @property
    def W(self) -> torch.Tensor:
        """W [R, V] as a view of Wt."""
        return self.Wt.t()


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _target_rows(workload: str, rows: int, V: int, g: torch.Generator, device) -> torch.Tensor:
    """fp32 target logits for `rows` rows of a workload."""
    x = torch.randn(rows, V, generator=g, device=device) * 3.0
    if workload == "tiny":
        ids = torch.randint(0, V, (rows, 1), generator=g, device=device)
        x.scatter_add_(1, ids, torch.full((rows, 1), 8.0, device=device))
    elif workload == "batched":
        for r in range(rows):
            k = int(torch.randint(1, 4, (1,), generator=g, device=device).item())
            ids = torch.randperm(V, generator=g, device=device)[:k]
            boost = 6.0 + 4.0 * torch.rand(k, generator=g, device=device)
            x[r, ids] += boost
    elif workload in ("headline", "block"):
        table = -1.1 * torch.log(torch.arange(1, V + 1, device=device, dtype=torch.float32))
        keys = torch.rand(rows, V, generator=g, device=device)
        perm = torch.argsort(keys, dim=1, stable=True)     # a random permutation per row
        x += table[perm]
    return x


def _gumbel_argmax(logits_over_T: torch.Tensor, g: torch.Generator) -> torch.Tensor:
    u = torch.rand(logits_over_T.shape, generator=g, device=logits_over_T.device)
    u = u.clamp_(min=1e-12, max=1.0 - 1e-7)
    return torch.argmax(logits_over_T - torch.log(-torch.log(u)), dim=-1)


def make_verify_inputs(workload: str, device="cpu", B: Optional[int] = None, gamma: Optional[int] = None,
                       V: Optional[int] = None, noise: Optional[float] = None,
                       row_block: int = 256, seed: Optional[int] = None) -> VerifyInputs:
    """Target / draft logits and draft tokens of a verification workload
    ("tiny", "batched", "headline" or "block").

    seed (default: the workload's) seeds the logit noise; another value gives
    an independent batch of the same recipe."""
    c = WORKLOADS[workload]
    B = c["B"] if B is None else B
    gamma = c["gamma"] if gamma is None else gamma
    V = c["V"] if V is None else V
    T = c["T"]
    dt = c["dtype"]
    sd = noise if noise is not None else (1.5 if workload == "batched" else 1.0)
    g = _gen(device, c["seed"] if seed is None else seed)
    gd = _gen(device, DRAFT_SEED)
    p = torch.empty(B, gamma + 1, V, dtype=dt, device=device)
    q = torch.empty(B, max(gamma, 0), V, dtype=dt, device=device)
    draft = torch.empty(B, max(gamma, 0), dtype=torch.int32, device=device)
    per = max(1, row_block // (gamma + 1))
    for b0 in range(0, B, per):
        b1 = min(B, b0 + per)
        nb = b1 - b0
        t = _target_rows(workload, nb * (gamma + 1), V, g, device).view(nb, gamma + 1, V)
        p[b0:b1] = t.to(dt)
        if gamma > 0:
            d = t[:, :gamma] + sd * torch.randn(nb, gamma, V, generator=g, device=device)
            qd = d.to(dt)
            q[b0:b1] = qd
            draft[b0:b1] = _gumbel_argmax(qd.float() / T, gd).to(torch.int32)
        del t
    conf = None
    if workload == "block" and gamma > 0:
        gc = _gen(device, c["conf_seed"])
        mu = 0.35 + 0.60 * torch.rand(B, 1, generator=gc, device=device)
        decay = 1.0 - 0.03 * torch.arange(gamma, device=device, dtype=torch.float32)[None, :]
        conf = (mu * decay + 0.05 * torch.randn(B, gamma, generator=gc, device=device)).clamp_(0.0, 1.0)
    return VerifyInputs(workload, B, gamma, V, T, p, q, draft, conf)


def sts_temperatures(gamma: int) -> list:
    """Per-position temperatures of the temperature-scaled workload-5 variant."""
    return [1.0 + 0.15 * i for i in range(gamma)]


def sts_head_logits(conf: torch.Tensor, temps) -> torch.Tensor:
    """Raw (over-confident) head log-odds [B, gamma] fp32 whose calibrated
    estimates are `conf` (see the module docstring)."""
    c = conf.double().clamp(1e-6, 1.0 - 1e-6)
    t = torch.tensor(list(temps), dtype=torch.float64, device=conf.device)[None, :]
    return (t * torch.log(c / (1.0 - c))).float().contiguous()


def make_markov_inputs(device="cpu", B: Optional[int] = None, gamma: Optional[int] = None,
                       V: Optional[int] = None, R: Optional[int] = None, uw_std: float = 0.02,
                       row_block: int = 256) -> MarkovInputs:
    """Backbone logits, Markov factors, anchors and target logits of the markov workload."""
    c = WORKLOADS["markov"]
    B = c["B"] if B is None else B
    gamma = c["gamma"] if gamma is None else gamma
    V = c["V"] if V is None else V
    R = c["R"] if R is None else R
    g = _gen(device, c["seed"])
    base = torch.empty(B, gamma, V, dtype=torch.bfloat16, device=device)
    p = torch.empty(B, gamma + 1, V, dtype=torch.bfloat16, device=device)
    per = max(1, row_block // (gamma + 1))
    for b0 in range(0, B, per):
        b1 = min(B, b0 + per)
        nb = b1 - b0
        bf = torch.randn(nb, gamma, V, generator=g, device=device) * 3.0
        base[b0:b1] = bf.to(torch.bfloat16)
        p[b0:b1, :gamma] = (bf + torch.randn(nb, gamma, V, generator=g, device=device)).to(torch.bfloat16)
        p[b0:b1, gamma] = (torch.randn(nb, V, generator=g, device=device) * 3.0).to(torch.bfloat16)
    U = (torch.randn(V, R, generator=g, device=device) * uw_std).to(torch.bfloat16)
    Wt = (torch.randn(V, R, generator=g, device=device) * uw_std).to(torch.bfloat16)
    x0 = torch.randint(0, V, (B,), generator=g, device=device).to(torch.int32)
    return MarkovInputs(B, gamma, V, R, c["T"], base, U, Wt, x0, p)


def tree_parents(branches: int = 4, depth: int = 5) -> list:
    """Parents (node m at index m-1) of `branches` chains of `depth` nodes
    hanging from the root."""
    par = []
    for k in range(branches):
        first = k * depth + 1
        par.append(0)
        par.extend(range(first, first + depth - 1))
    return par


@dataclass
class TreeInputs:
    B: int
    V: int
    T: float
    parents: list
    p: torch.Tensor         # [B, N+1, V]
    q: torch.Tensor         # [B, NQ, V]
    tokens: torch.Tensor    # [B, N] int32


def make_tree_inputs(device="cpu", B: int = 64, V: int = 129280, parents: Optional[list] = None,
                     dtype=torch.bfloat16, noise: float = 1.0, seed: int = 1007, row_block: int = 256,
                     T: float = 1.0) -> TreeInputs:
    """Target / draft logits and node tokens of the tree-verification workload."""
    par = tree_parents() if parents is None else list(parents)
    N = len(par)
    internal = sorted(set(par))
    qidx = {n: j for j, n in enumerate(internal)}
    g = _gen(device, seed)
    gd = _gen(device, DRAFT_SEED)
    p = torch.empty(B, N + 1, V, dtype=dtype, device=device)
    q = torch.empty(B, len(internal), V, dtype=dtype, device=device)
    tokens = torch.empty(B, N, dtype=torch.int32, device=device)
    per = max(1, row_block // (N + 1))
    for b0 in range(0, B, per):
        b1 = min(B, b0 + per)
        nb = b1 - b0
        t = _target_rows("headline", nb * (N + 1), V, g, device).view(nb, N + 1, V)
        p[b0:b1] = t.to(dtype)
        if internal:
            d = t[:, internal] + noise * torch.randn(nb, len(internal), V, generator=g, device=device)
            qd = d.to(dtype)
            q[b0:b1] = qd
            for m in range(1, N + 1):
                tokens[b0:b1, m - 1] = _gumbel_argmax(qd[:, qidx[par[m - 1]]].float() / T, gd).to(torch.int32)
        del t
    return TreeInputs(B, V, T, par, p, q, tokens)


def make_rnn_recurrence(R: int, device="cpu", std: Optional[float] = None, seed: int = 1006) -> torch.Tensor:
    """Recurrent matrix A [R, R] bf16 of the RNN-head variant of the markov workload."""
    g = _gen(device, seed)
    sd = 0.9 / (R ** 0.5) if std is None else std
    return (torch.randn(R, R, generator=g, device=device) * sd).to(torch.bfloat16)


def bytes_single_read(inp: VerifyInputs) -> int:
    """Bytes of every logit row read once (the row-statistics pass)."""
    es = inp.p.element_size()
    return inp.B * ((inp.gamma + 1) + inp.gamma) * inp.V * es


def describe(workload: str) -> str:
    c = WORKLOADS[workload]
    return f"{workload}: B={c['B']} gamma={c['gamma']} V={c['V']} {str(c['dtype']).split('.')[-1]} T={c['T']}"


__all__ = ["WORKLOADS", "VERIFY_SEED", "DRAFT_SEED", "VerifyInputs", "MarkovInputs", "make_verify_inputs",
           "make_markov_inputs", "make_rnn_recurrence", "TreeInputs", "make_tree_inputs", "tree_parents", "sts_temperatures", "sts_head_logits", "bytes_single_read",
           "describe"]
