"""Pins for the oracle's ELB counters and gather maps (integer work).

Checked against library routines (bincount, stable argsort, cumsum) and the
permutation invariants: every pair lands in exactly one sorted row, gather
followed by scatter is the identity, counter sums equal T*k per layer.
"""
import numpy as np
import pytest

import oracle
import synth


def _ids(T, k, E, seed):
    rng = np.random.default_rng(seed)
    # distinct experts per token, like a top-k
    rows = [rng.permutation(E)[:k] for _ in range(T)]
    return np.array(rows, dtype=np.int32).reshape(T, k)


@pytest.mark.parametrize("T,k,E", [(4, 2, 8), (16, 6, 64), (17, 4, 60), (1, 2, 16), (0, 3, 8)])
def test_elb_counts_are_bincount(T, k, E):
    L = 3
    ids = _ids(T, k, E, T + E).reshape(T, k)
    c = np.zeros((L, E), np.int32)
    c = oracle.elb_update(c, ids, 1)
    assert np.array_equal(c[1], np.bincount(ids.ravel(), minlength=E))
    assert c[1].sum() == T * k
    assert c[0].sum() == 0 and c[2].sum() == 0
    c2 = oracle.elb_update(c, ids, 1)            # accumulates
    assert np.array_equal(c2[1], 2 * c[1])


def test_elb_chunk_rows_sum():
    # 16 draft steps at T = 1, top-4, 24 layers: each layer's row sums to 64
    L, E, k = 24, 60, 4
    c = np.zeros((L, E), np.int32)
    for step in range(16):
        for layer in range(L):
            c = oracle.elb_update(c, _ids(1, k, E, step * 100 + layer), layer)
    assert np.all(c.sum(axis=1) == 16 * k)


def test_elb_ignores_out_of_range():
    c = oracle.elb_update(np.zeros((1, 4), np.int32), np.array([[0, 4], [-1, 3]]), 0)
    assert c.tolist() == [[1, 0, 0, 1]]


@pytest.mark.parametrize("T,k,E", [(4, 2, 8), (16, 6, 64), (17, 4, 60), (9, 4, 60), (1, 6, 64),
                                   (33, 8, 9)])
def test_gather_maps_invariants(T, k, E):
    ids = _ids(T, k, E, 7 * T + E)
    m = oracle.gather_maps(ids, E)
    flat = ids.ravel()
    n = T * k
    # offsets: exclusive prefix sum of the per-expert counts
    cnt = np.bincount(flat, minlength=E)
    assert np.array_equal(m["offsets"], np.concatenate([[0], np.cumsum(cnt)]))
    # stable counting sort == library stable argsort
    assert np.array_equal(m["sorted_pair"], np.argsort(flat, kind="stable"))
    # permutation and inverse
    sp, pp = m["sorted_pair"], m["pair_pos"]
    assert sorted(sp.tolist()) == list(range(n))
    assert np.array_equal(sp[pp], np.arange(n))
    assert np.array_equal(pp[sp], np.arange(n))
    # experts non-decreasing along rows, pairs increasing within an expert
    ex = flat[sp]
    assert np.all(np.diff(ex) >= 0)
    for e in range(E):
        r0, r1 = m["offsets"][e], m["offsets"][e + 1]
        assert np.all(np.diff(sp[r0:r1]) > 0)
        assert np.all(flat[sp[r0:r1]] == e)
    assert np.array_equal(m["sorted_token"], sp // k)
    act = np.nonzero(cnt)[0]
    assert m["n_active"] == len(act)
    assert np.array_equal(m["active"][:len(act)], act)
    assert np.all(m["active"][len(act):] == -1)
    # gather then scatter is the identity on row data
    rows = np.arange(n) * 10 + 3
    gathered = rows[sp]
    back = np.empty_like(rows)
    back[sp] = gathered
    assert np.array_equal(back, rows)
    assert np.array_equal(gathered[pp], rows)


def test_gather_hand_example():
    # T = 3, k = 2: pairs 0..5 -> experts [2,0 | 1,2 | 0,2]
    ids = np.array([[2, 0], [1, 2], [0, 2]], np.int32)
    m = oracle.gather_maps(ids, 4)
    assert m["offsets"].tolist() == [0, 2, 3, 6, 6]
    assert m["sorted_pair"].tolist() == [1, 4, 2, 0, 3, 5]
    assert m["sorted_token"].tolist() == [0, 2, 1, 0, 1, 2]
    assert m["pair_pos"].tolist() == [3, 0, 2, 4, 1, 5]
    assert m["active"].tolist() == [0, 1, 2, -1]
    assert int(m["n_active"]) == 3


def test_gather_drops_out_of_range():
    ids = np.array([[1, 5], [0, -2]], np.int32)
    m = oracle.gather_maps(ids, 3)
    assert m["offsets"].tolist() == [0, 1, 2, 2]
    assert m["pair_pos"].tolist() == [1, -1, 0, -1]
    assert m["sorted_pair"][:2].tolist() == [2, 0]


def test_token_stream_correlation():
    """The AR(1) token stream: unit marginals, lag-one correlation rho,
    independent rows at rho = 0 (input generator only)."""
    s = synth.QWEN_CHUNK
    for rho in (0.0, 0.8):
        x = synth.token_stream(s, 400, rho).astype(np.float64)
        assert abs(x.std() - 1.0) < 0.02
        c = np.mean(np.sum(x[1:] * x[:-1], axis=1) / s.H)
        assert abs(c - rho) < 0.02
