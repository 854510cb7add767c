"""Pins for the oracle's 2- and 8-bit GPTQ-layout dequantisation and the
draft FFN at those widths (the 2/8-bit draft precisions the pages compare).

Words are packed by hand here (not with the synthetic packer), values are
worked out by hand (tests/golden/gptq_dequant_2_8bit_closed_form.json), and
the FFN is held to the same identities as the 4-bit one: grouped by expert
equals every expert on every token then masked, and equals the per-token
ordering.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _word(codes, bits):
    """Hand packing: codes (low code first) -> uint32 word."""
    w = 0
    for i, v in enumerate(codes):
        w |= (int(v) & ((1 << bits) - 1)) << (bits * i)
    return np.uint32(w)


@pytest.mark.parametrize("bits", [2, 8])
def test_code_order_and_groups(bits):
    per = 32 // bits
    K, N = 256, 32
    qw = np.zeros((K // per, N), np.uint32)
    r, n, i = 3, 5, per - 2
    code = (1 << bits) - 2
    qw[r, n] = np.uint32(code) << np.uint32(bits * i)     # one code: row per*r + i
    s = np.empty((K // 128, N), np.float16)
    s[0], s[1] = 1.0, 0.25
    qz = np.zeros((K // 128, N // per), np.uint32)
    W = oracle.dequant_gptq(qw.view(np.int32), s, qz.view(np.int32), bits=bits)
    assert np.argwhere(W != 0).tolist() == [[per * r + i, n]]
    assert W[per * r + i, n] == code
    # the same code in the second group (rows 128..255) takes its scale
    qw2 = np.zeros_like(qw)
    qw2[128 // per + r, n] = np.uint32(code) << np.uint32(bits * i)
    W2 = oracle.dequant_gptq(qw2.view(np.int32), s, qz.view(np.int32), bits=bits)
    assert np.argwhere(W2 != 0).tolist() == [[128 + per * r + i, n]]
    assert W2[128 + per * r + i, n] == code * 0.25


@pytest.mark.parametrize("bits", [2, 8])
def test_zero_order(bits):
    per = 32 // bits
    K, N = 128, 2 * per
    qw = np.zeros((K // per, N), np.uint32)
    qz = np.zeros((1, N // per), np.uint32)
    zval = (1 << bits) - 1
    qz[0, 1] = np.uint32(zval) << np.uint32(bits * 3)    # zero of column per + 3
    s = np.ones((1, N), np.float16)
    W = oracle.dequant_gptq(qw.view(np.int32), s, qz.view(np.int32), bits=bits)
    assert np.all(W[:, per + 3] == -zval)
    W[:, per + 3] = 0
    assert np.all(W == 0)


@pytest.mark.parametrize("bits", [2, 8])
def test_all_code_zero_pairs(bits):
    per = 32 // bits
    L = 1 << bits
    K, N = 128, L * L if bits == 2 else 256
    q = np.zeros((K, N), np.uint8)
    z = np.zeros((1, N), np.uint8)
    for n in range(N):
        if bits == 2:
            q[:, n], z[0, n] = n % L, n // L          # all 16 (q, z) pairs
        else:
            q[:, n], z[0, n] = n, 255 - n             # every code and every zero
    qw = np.zeros((K // per, N), np.uint32)
    for rr in range(K // per):
        for n in range(N):
            qw[rr, n] = _word(q[per * rr:per * rr + per, n], bits)
    qz = np.zeros((1, N // per), np.uint32)
    for c in range(N // per):
        qz[0, c] = _word(z[0, per * c:per * c + per], bits)
    uq, uz = oracle.unpack_gptq(qw.view(np.int32), qz.view(np.int32), bits)
    assert np.array_equal(uq, q) and np.array_equal(uz, z)
    W = oracle.dequant_gptq(qw.view(np.int32), np.ones((1, N), np.float16),
                            qz.view(np.int32), bits=bits)
    assert np.array_equal(W[0], q[0].astype(np.float64) - z[0].astype(np.float64))


def test_golden_fixture():
    with open(os.path.join(GOLDEN, "gptq_dequant_2_8bit_closed_form.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        bits = case["bits"]
        per = 32 // bits
        K, N = 128, per
        qw = np.zeros((K // per, N), np.uint32)
        qw[0, 0] = np.uint32(int(case["qword"], 16))
        qz = np.zeros((1, 1), np.uint32)
        qz[0, 0] = np.uint32(int(case["zword"], 16))
        s = np.full((1, N), case["scale"], np.float16)
        W = oracle.dequant_gptq(qw.view(np.int32), s, qz.view(np.int32), bits=bits)
        assert W[:per, 0].tolist() == case["expected_col0"], case["derivation"]


@pytest.mark.parametrize("bits", [2, 8])
def test_rtn_error_bound_and_exact_fp32(bits):
    rng = np.random.default_rng(bits)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float16)
    qw, s, qz = synth.gptq_from_linear(w, bits)
    W = oracle.dequant_gptq(qw, s, qz, bits=bits)
    sg = np.repeat(s.astype(np.float64), 128, axis=0)
    # half a step, plus the grid's end moving by qmax times the fp16 rounding
    # of the step (at most 2^-11 relative) where the top code clips
    qmax = (1 << bits) - 1
    bound = (0.5 + qmax * 2.0 ** -11 * 1.001 + 1e-3) * sg
    assert np.all(np.abs(W - w.T.astype(np.float64)) <= bound)
    W32 = oracle.dequant_gptq(qw, s, qz, dtype=np.float32, bits=bits).astype(np.float64)
    assert np.array_equal(W32, W)


def _layer(seed, bits, E=6, H=256, I=128):
    rng = np.random.default_rng(seed)
    q = []
    for _ in range(E):
        w13 = (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float16)
        w2 = (rng.standard_normal((H, I)) * 0.02).astype(np.float16)
        q.append(synth.expert_int4(w13, w2, bits))
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float16)
    return q, wr


@pytest.mark.parametrize("bits", [2, 8])
def test_grouped_equals_masked_brute_force_and_per_token(bits):
    kind = f"int{bits}"
    q, wr = _layer(bits, bits)
    E, k, T = 6, 2, 7
    x = np.random.default_rng(9).standard_normal((T, 256)).astype(np.float16)
    r = oracle.route_topk(x, wr, k)
    m = oracle.gather_maps(r["ids"], E)
    y = oracle.grouped_ffn(x, m, q, kind)
    allout = np.stack([oracle.expert_ffn_int4(x, q[e]["w13"], q[e]["w2"], bits=bits)
                       for e in range(E)])
    pt = oracle.per_token_ffn(x, r["ids"], q, kind)
    for p in range(T * k):
        t, e = p // k, int(r["ids"].ravel()[p])
        assert np.allclose(y[m["pair_pos"][p]], allout[e, t], rtol=1e-12, atol=1e-14)
        assert np.max(np.abs(y[m["pair_pos"][p]] - pt[t, p % k])) <= \
            1e-12 * max(1.0, np.max(np.abs(pt[t, p % k])))


def test_widths_differ_and_converge():
    # the same fp16 expert at 2, 4 and 8 bits: each wider code shrinks the
    # dequantisation error (finer grids)
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((128, 256)) * 0.02).astype(np.float16)
    errs = []
    for bits in (2, 4, 8):
        W = oracle.dequant_gptq(*synth.gptq_from_linear(w, bits), bits=bits)
        errs.append(np.abs(W - w.T.astype(np.float64)).mean())
    assert errs[0] > errs[1] > errs[2]
