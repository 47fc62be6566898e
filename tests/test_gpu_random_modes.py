"""Seeded random configurations of the two-stage dispatch and the FIFO ring
dispatch through the C ABI, with the same checks as their own test files
(control-plane state after each call from the oracle, staged rows, gathered
rows, every output element): dense and expert routes, ragged row counts, both
tile widths, a random self shard (or none), and for the ring a random number of
rings per shard and slots per ring. Every case is drawn from a fixed seed."""
import numpy as np
import pytest

from fg_harness import dense_case, ep_case, log
import test_gpu_ring as ring_mode
import test_gpu_two_stage as two_stage_mode

pytestmark = pytest.mark.gpu


def _case(seed, rng):
    kind = ["contig", "perm", "ep"][seed % 3]
    K = int(rng.choice([128, 256, 640, 1024]))
    tile_n = int(rng.choice([128, 256]))
    N = tile_n * int(rng.integers(1, 4))
    S = int(rng.integers(1, 7))
    if kind == "ep":
        case = ep_case(seed, S, int(rng.integers(1, 300)), K, N, n_experts=int(rng.choice([8, 16])),
                       topk=int(rng.integers(1, 4)), n_local=int(rng.choice([2, 4, 8])))
    else:
        case = dense_case(seed, S, int(rng.integers(1, 900)), K, N,
                          gather="permutation" if kind == "perm" else "contiguous")
    return kind, S, K, N, tile_n, case


@pytest.mark.parametrize("seed", list(range(300, 316)))
def test_random_dispatch_mode(seed):
    rng = np.random.default_rng(seed)
    kind, S, K, N, tile_n, case = _case(seed, rng)
    self_shard = int(rng.integers(-1, S))
    if seed % 2 == 0:
        log(f"seed {seed}: two-stage {kind} S={S} K={K} N={N} tile_n={tile_n} self={self_shard}")
        two_stage_mode._run(case, 2, self_shard=self_shard, ctx_kw=dict(tile_n=tile_n))
    else:
        n_channels, ring_chunks = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        log(f"seed {seed}: ring {kind} S={S} K={K} N={N} tile_n={tile_n} self={self_shard} "
            f"rings/shard={n_channels} slots={ring_chunks}")
        ring_mode._run(case, 2, n_channels=n_channels, ring_chunks=ring_chunks, self_shard=self_shard,
                       ctx_kw=dict(tile_n=tile_n))
