"""Pins for the oracle's routing (logits, top-k, softmax weights, shared gate).

The expected values here come from closed forms worked out by hand, from
brute force over all k-subsets, and from the fp64 dot product within the
classical summation error bound -- never from the oracle itself.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth


def f16(a):
    return np.asarray(a, dtype=np.float16)


# ---------------------------------------------------------------- logits ----

def test_logit_unit_vector_picks_weight():
    rng = np.random.default_rng(1)
    H, E = 512, 5
    w = f16(rng.standard_normal((E, H)) * 0.02)
    for h in (0, 7, 8, 63, 64, 511):
        x = np.zeros((1, H), np.float16)
        x[0, h] = 1.0
        L = oracle.logits_pinned_f32(x, w)
        assert np.array_equal(L[0], w[:, h].astype(np.float32))


def test_logit_exact_sum_of_powers_of_two():
    H = 2048
    x = np.ones((1, H), np.float16)
    w = np.full((3, H), 2.0 ** -10, np.float16)
    L = oracle.logits_pinned_f32(x, w)
    assert np.all(L == np.float32(H * 2.0 ** -10))


def _big_plus_ones(H, ones_at):
    x = np.zeros((1, H), np.float16)
    w = np.zeros((1, H), np.float16)
    x[0, 0] = 4096.0
    w[0, 0] = 4096.0           # product 2**24: adding 1 to it rounds back
    for h in ones_at:
        x[0, h] = 1.0
        w[0, h] = 1.0
    return x, w


def test_pinned_order_sequential_within_lane():
    # lane 0 owns chunk 0 (h = 0..7).  In order: 2^24 + 1 -> 2^24 (ties to
    # even), seven times.  Summing the ones first would give 2^24 + 8.
    x, w = _big_plus_ones(512, range(1, 8))
    assert oracle.logits_pinned_f32(x, w)[0, 0] == np.float32(2.0 ** 24)


def test_pinned_order_chunk_ownership():
    # H = 1024: chunk 64 (h = 512..519) belongs to lane 0 again (64 mod 64),
    # after chunk 0, so both ones are absorbed: 2^24.  Were chunk 64 owned by
    # any lane other than 0, the butterfly would add 2 to 2^24 exactly.
    x, w = _big_plus_ones(1024, (512, 513))
    assert oracle.logits_pinned_f32(x, w)[0, 0] == np.float32(2.0 ** 24)


def test_pinned_order_butterfly():
    # ones in lanes 1 and 3 (chunks 1 and 3 -> h = 8 and h = 24).  Butterfly:
    # distance 2 gives lane 1 the value 1 + 1 = 2, distance 1 gives lane 0
    # 2^24 + 2 (exact, even).  A left-to-right sum over lanes would give 2^24.
    x, w = _big_plus_ones(512, (8, 24))
    assert oracle.logits_pinned_f32(x, w)[0, 0] == np.float32(2.0 ** 24 + 2)


@pytest.mark.parametrize("H", [256, 2048, 4096])
def test_pinned_logits_within_summation_bound(H):
    rng = np.random.default_rng(H)
    x = f16(rng.standard_normal((4, H)))
    w = f16(rng.standard_normal((7, H)) * 0.02)
    L32 = oracle.logits_pinned_f32(x, w).astype(np.float64)
    xd = x.astype(np.float64)
    wd = w.astype(np.float64)
    exact = xd @ wd.T
    absum = np.abs(xd) @ np.abs(wd).T
    n = (H // 8 + 63) // 64 * 8 + 6          # additions along any path
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    assert np.all(np.abs(L32 - exact) <= gamma * absum)


# ----------------------------------------------------------------- top-k ----

def _brute_topk(L, k):
    E = L.shape[0]
    best, best_set = None, None
    for s in itertools.combinations(range(E), k):      # lexicographic order
        v = sum(float(L[i]) for i in s)
        if best is None or v > best:
            best, best_set = v, s
    return set(best_set)


@pytest.mark.parametrize("E,k", [(8, 2), (12, 4), (6, 6), (5, 1)])
def test_topk_matches_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    H = 256
    x = f16(rng.standard_normal((6, H)))
    w = f16(rng.standard_normal((E, H)) * 0.02)
    r = oracle.route_topk(x, w, k)
    L = r["logits32"]
    for t in range(x.shape[0]):
        assert set(r["ids"][t].tolist()) == _brute_topk(L[t].astype(np.float64), k)
        # rank order: logits non-increasing along the slots
        v = L[t, r["ids"][t]]
        assert np.all(v[:-1] >= v[1:])


def test_topk_ties_lower_index_first():
    E, k, H = 8, 3, 256
    x = np.zeros((2, H), np.float16)
    w = f16(np.random.default_rng(0).standard_normal((E, H)))
    r = oracle.route_topk(x, w, k)
    assert r["ids"].tolist() == [[0, 1, 2], [0, 1, 2]]
    assert np.allclose(r["weights"], 1.0 / E, rtol=0, atol=1e-15)
    # partial tie: experts 2 and 5 share the best logit, 1 and 6 the next
    w = np.zeros((E, H), np.float16)
    w[2, 0] = w[5, 0] = 1.0
    w[1, 0] = w[6, 0] = 0.5
    x = np.zeros((1, H), np.float16)
    x[0, 0] = 1.0
    r = oracle.route_topk(x, w, 4)
    assert r["ids"][0].tolist() == [2, 5, 1, 6]


def test_topk_monotone_router():
    E, k, H = 16, 4, 256
    w = np.zeros((E, H), np.float16)
    w[:, 0] = f16(np.arange(E) / 64.0)
    x = np.zeros((1, H), np.float16)
    x[0, 0] = 1.0
    r = oracle.route_topk(x, w, k)
    assert r["ids"][0].tolist() == [15, 14, 13, 12]


def test_softmax_weights_closed_form():
    # two experts with logits ln 3 and 0, the rest -inf-like far below:
    # softmax gives 3/4 and 1/4 (up to the others' tiny mass).
    E, H = 4, 256
    w = np.zeros((E, H), np.float16)
    w[0, 0] = 1.0
    x = np.zeros((1, H), np.float16)
    x[0, 0] = np.log(3.0)
    r = oracle.route_topk(x, w, 2)
    l3 = float(np.float16(np.log(3.0)))
    e = np.exp(l3)
    assert r["ids"][0].tolist() == [0, 1]
    assert abs(r["weights"][0, 0] - e / (e + 3)) < 1e-15
    assert abs(r["weights"][0, 1] - 1 / (e + 3)) < 1e-15
    rr = oracle.route_topk(x, w, 2, renormalize=True)
    assert abs(rr["weights"][0].sum() - 1) < 1e-15
    assert abs(rr["weights"][0, 0] - e / (e + 1)) < 1e-15


def test_softmax_sums_to_one_over_all_experts():
    rng = np.random.default_rng(5)
    x = f16(rng.standard_normal((3, 512)))
    w = f16(rng.standard_normal((9, 512)) * 0.02)
    r = oracle.route_topk(x, w, 9)
    assert np.allclose(r["weights"].sum(axis=1), 1.0, atol=1e-12)


def test_shared_gate_sigmoid():
    H = 256
    x = np.zeros((2, H), np.float16)
    x[1, 3] = 2.0
    g = np.zeros(H, np.float16)
    g[3] = 1.0
    w = f16(np.random.default_rng(2).standard_normal((4, H)))
    r = oracle.route_topk(x, w, 2, w_shared_gate=g)
    assert r["gate"][0] == 0.5
    assert abs(r["gate"][1] - 1.0 / (1.0 + np.exp(-2.0))) < 1e-15


def test_draft_and_verify_routing_identical():
    # The draft reuses the target's router tensor, so on the same tokens the
    # two paths route identically (same function, same input).
    shape = synth.TINY
    wr = synth.router(shape)
    x = synth.tokens(shape, 4)
    a = oracle.route_topk(x, wr, shape.k)
    b = oracle.route_topk(x.copy(), wr.copy(), shape.k)
    assert np.array_equal(a["ids"], b["ids"])
