"""Seeded synthetic inputs for the fused gather-GEMM and the protocol stress run.

This module only draws random inputs (activations, weights, permutations, top-k
expert choices, stress chunk sizes and producer delays). It holds none of the
method's arithmetic: no layout, no gather, no counts, no GEMM. Both the HIP path
and the CPU oracle consume exactly the bytes produced here.

Every draw uses ``torch.Generator(device="cpu").manual_seed(seed)``; floating
point draws are float32 rounded to bfloat16 with round-to-nearest-even. "N(0, s)"
means a normal distribution with standard deviation ``s``.

Weight layout: the logical weight is K x N (rows = contraction index). It is
stored with the contraction index contiguous, i.e. as an [N, K] row-major array
(the storage of a linear layer's weight), and per expert as [G, N, K].
"""
from __future__ import annotations

import dataclasses

import torch

CHUNK_ROWS = 64
ROW_BLOCK = 128


@dataclasses.dataclass
class DenseInputs:
    shards: list          # n_shards x bf16 [rows, K]
    w: torch.Tensor       # bf16 [N, K]  (logical W is [K, N])
    perm: torch.Tensor | None  # int32 [n_shards*rows] destination of stream row s*rows+i, or None
    sigma_x: float
    sigma_w: float


@dataclasses.dataclass
class EPInputs:
    shards: list          # n_shards x bf16 [tokens, K]
    topk: torch.Tensor    # int32 [n_shards, tokens, topk] distinct experts per token
    w: torch.Tensor       # bf16 [n_local, N, K]
    expert_base: int
    n_local: int
    sigma_x: float
    sigma_w: float


@dataclasses.dataclass
class StressInputs:
    chunk_rows: torch.Tensor   # int32 [P, C, KC]; 0 = inactive slot, else rows in [1, 64]
    delays_ns: torch.Tensor    # int32 [iters, P, C, KC]; producer delay before each chunk


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _normal_bf16(g, shape, std):
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def dense_inputs(seed: int, n_shards: int, rows: int, K: int, N: int, *,
                 gather: str = "contiguous", sigma_x: float = 1.0,
                 sigma_w: float = 0.02) -> DenseInputs:
    """Shards ~N(0, sigma_x), W ~N(0, sigma_w); ``gather`` is 'contiguous' or 'permutation'."""
    g = _gen(seed)
    shards = [_normal_bf16(g, (rows, K), sigma_x) for _ in range(n_shards)]
    w = _normal_bf16(g, (N, K), sigma_w)
    perm = None
    if gather == "permutation":
        perm = torch.randperm(n_shards * rows, generator=g).to(torch.int32)
    elif gather != "contiguous":
        raise ValueError(gather)
    return DenseInputs(shards, w, perm, sigma_x, sigma_w)


def ep_inputs(seed: int, n_shards: int = 8, tokens: int = 1024, K: int = 7168,
              N: int = 2048, n_experts: int = 64, topk: int = 8, n_local: int = 8,
              expert_base: int = 0, sigma_x: float = 1.0,
              sigma_w: float = 0.02) -> EPInputs:
    """Top-k routing: each token picks ``topk`` distinct experts uniformly out of
    ``n_experts``; this GPU owns experts [expert_base, expert_base + n_local)."""
    g = _gen(seed)
    shards = [_normal_bf16(g, (tokens, K), sigma_x) for _ in range(n_shards)]
    scores = torch.rand(n_shards * tokens, n_experts, generator=g)
    choice = torch.argsort(scores, dim=1)[:, :topk].to(torch.int32)
    topk_t = choice.reshape(n_shards, tokens, topk).contiguous()
    w = _normal_bf16(g, (n_local, N, K), sigma_w)
    return EPInputs(shards, topk_t, w, expert_base, n_local, sigma_x, sigma_w)


def combine_inputs(seed: int, rows: int, N: int, n_shards: int, tokens: int, topk: int,
                   sigma: float = 1.0):
    """Inputs of the combine step: expert outputs bf16 [rows, N] ~N(0, sigma) in
    gathered-row order, and gate weights fp32 [n_shards, tokens, topk] drawn
    U(0, 1) and normalised to sum 1 over each token's top-k list."""
    g = _gen(seed)
    out = _normal_bf16(g, (rows, N), sigma)
    u = torch.rand(n_shards, tokens, topk, generator=g, dtype=torch.float32)
    w = (u / u.sum(dim=-1, keepdim=True)).contiguous()
    return out, w


def stress_inputs(seed: int, producers: int = 64, consumers: int = 64,
                  max_chunks: int = 4, signals: int = 10000, iters: int = 50,
                  max_delay_ns: int = 20000) -> StressInputs:
    """Active slot set: every (producer, consumer) pair gets 2 chunks, a seeded
    choice of pairs gets a 3rd, so that the active count equals ``signals``;
    the last chunk of each pair has a seeded row count in [1, 64], the others 64.
    Delays are uniform integers in [0, max_delay_ns] per (iteration, slot)."""
    g = _gen(seed)
    pairs = producers * consumers
    base = 2 * pairs
    extra = signals - base
    if not (0 <= extra <= pairs * (max_chunks - 2)):
        raise ValueError("signals not reachable with this slot capacity")
    n_chunks = torch.full((pairs,), 2, dtype=torch.int32)
    if extra:
        pick = torch.randperm(pairs, generator=g)[:extra]
        n_chunks[pick] += 1
    rows = torch.zeros(pairs, max_chunks, dtype=torch.int32)
    last_rows = torch.randint(1, CHUNK_ROWS + 1, (pairs,), generator=g, dtype=torch.int32)
    for k in range(max_chunks):
        full = (k < n_chunks - 1)
        last = (k == n_chunks - 1)
        rows[:, k] = torch.where(full, torch.full_like(last_rows, CHUNK_ROWS),
                                 torch.where(last, last_rows, torch.zeros_like(last_rows)))
    chunk_rows = rows.reshape(producers, consumers, max_chunks).contiguous()
    delays = torch.randint(0, max_delay_ns + 1, (iters, producers, consumers, max_chunks),
                           generator=g, dtype=torch.int32)
    return StressInputs(chunk_rows, delays)


# Named workloads with the sizes, distributions and structure of the five
# configurations the method is measured on.
CONFIGS = {
    "tiny": dict(kind="dense", seed=1001, n_shards=4, rows=256, K=256, N=512,
                 gather="contiguous", iters=3),
    "tp": dict(kind="dense", seed=1002, n_shards=4, rows=2048, K=4096, N=4096,
               gather="contiguous", iters=20),
    "ep": dict(kind="ep", seed=1003, n_shards=8, tokens=1024, K=7168, N=2048,
               n_experts=64, topk=8, n_local=8, expert_base=0, iters=20),
    "stress": dict(kind="stress", seed=1004, producers=64, consumers=64, max_chunks=4,
                   signals=10000, iters=50, max_delay_ns=20000),
    "large": dict(kind="dense", seed=1005, n_shards=8, rows=4096, K=8192, N=8192,
                  gather="permutation", iters=50),
}


def make(name: str, **overrides):
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    cfg.pop("iters", None)
    if kind == "dense":
        return dense_inputs(cfg.pop("seed"), cfg.pop("n_shards"), cfg.pop("rows"),
                            cfg.pop("K"), cfg.pop("N"), **cfg)
    if kind == "ep":
        return ep_inputs(cfg.pop("seed"), **cfg)
    if kind == "stress":
        return stress_inputs(cfg.pop("seed"), **cfg)
    raise ValueError(kind)
