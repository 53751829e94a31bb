"""bench.py's work convention, pinned to the products the method's definition contains.

The throughput figures count 12 Nq Nk d flops per head for the forward (30 for the reverse pass),
half when causal. Here the float64 oracle runs on a counting array type that adds 2 m k n for every
matrix product m x k @ k x n it performs: the forward definition (S, the two halves of the score
tangent, P V, dP V, P dV) and the reverse-pass steps (the three score products recomputed, then
twelve more) must add up to exactly bench.py's numbers, for several shapes.
"""
import numpy as np
import pytest

import bench
from oracle import oracle_bwd_head, oracle_fwd_head


class Counting(np.ndarray):
    flops = 0

    def __matmul__(self, other):
        a, b = np.asarray(self), np.asarray(other)
        Counting.flops += 2 * a.shape[0] * a.shape[1] * b.shape[1]
        return (a @ b).view(Counting)

    def __rmatmul__(self, other):
        a, b = np.asarray(other), np.asarray(self)
        Counting.flops += 2 * a.shape[0] * a.shape[1] * b.shape[1]
        return (a @ b).view(Counting)


def arrays(rng, Nq, Nk, d):
    c = lambda *s: rng.standard_normal(s).view(Counting)
    return c(Nq, d), c(Nk, d), c(Nk, d), c(Nq, d), c(Nk, d), c(Nk, d), c(Nq, d), c(Nq, d)


@pytest.mark.parametrize("Nq,Nk,d", [(5, 7, 3), (16, 16, 64), (9, 30, 8)])
def test_forward_and_reverse_product_counts(Nq, Nk, d):
    q, k, v, tq, tk, tv, go, gto = arrays(np.random.default_rng(Nq * Nk + d), Nq, Nk, d)
    bias = np.zeros((Nq, Nk)).view(Counting)
    Counting.flops = 0
    oracle_fwd_head(q, k, v, tq, tk, tv, bias, 0.5)
    assert Counting.flops == bench.fwd_flops(1, 1, Nq, Nk, d, False) == 12 * Nq * Nk * d
    Counting.flops = 0
    oracle_bwd_head(q, k, v, tq, tk, tv, go, gto, bias, 0.5)
    assert Counting.flops == bench.bwd_flops(1, 1, Nq, Nk, d, False) == 30 * Nq * Nk * d


def test_batches_heads_and_causal_halving():
    assert bench.fwd_flops(4, 16, 2048, 2048, 64, True) == 12 * 2048 * 2048 * 64 * 64 / 2 == 103079215104.0
    assert bench.bwd_flops(2, 3, 100, 50, 64, False) == 30 * 100 * 50 * 64 * 6
    assert bench.fwd_flops(2, 3, 100, 50, 64, True) * 2 == bench.fwd_flops(2, 3, 100, 50, 64, False)
    # the halving is the convention; the exact count of visible pairs (j <= i) is N(N+1)/2
    N = 2048
    assert abs(N * (N + 1) / 2 / (N * N) - 0.5) < 1e-3
