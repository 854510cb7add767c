"""Pins for the oracle's INT4 dequantisation, expert FFNs and combine.

Dequantisation is checked on hand-packed words with values worked out by
hand; the FFN on closed forms (zero weights, a one-hot input with known SiLU
values), on an evaluation order different from the oracle's (every expert on
every token, then a mask), on the pages' claim that grouping by expert equals
the per-token ordering, and on the two-shared-experts concatenation identity.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pack_words(nibbles_rows):
    """Hand packing for the tests: list of 8 nibbles -> uint32 word."""
    w = 0
    for i, v in enumerate(nibbles_rows):
        w |= (int(v) & 0xF) << (4 * i)
    return np.uint32(w)


def _mat(K, N, qnib, znib, scale):
    """qweight/scales/qzeros where every code is qnib and every zero znib."""
    qw = np.full((K // 8, N), _pack_words([qnib] * 8), np.uint32).view(np.int32)
    qz = np.full((K // 128, N // 8), _pack_words([znib] * 8), np.uint32).view(np.int32)
    s = np.full((K // 128, N), scale, np.float16)
    return qw, s, qz


def test_dequant_q_equals_z_is_zero():
    for q in range(16):
        W = oracle.dequant_gptq(*_mat(128, 8, q, q, 0.37))
        assert np.all(W == 0)


def test_dequant_full_scale():
    W = oracle.dequant_gptq(*_mat(256, 16, 15, 0, 2.0 ** -4))
    assert np.all(W == 0.9375)


def test_dequant_nibble_order_and_groups():
    K, N = 256, 16
    qw = np.zeros((K // 8, N), np.uint32)
    r, n, i = 5, 3, 6
    qw[r, n] = np.uint32(9) << np.uint32(4 * i)          # one code, row 8r+i
    s = np.empty((K // 128, N), np.float16)
    for g in range(K // 128):
        s[g] = 2.0 ** -g                                  # per-group scale
    qz = np.zeros((K // 128, N // 8), np.uint32)
    W = oracle.dequant_gptq(qw.view(np.int32), s, qz.view(np.int32))
    nz = np.argwhere(W != 0)
    assert nz.tolist() == [[8 * r + i, n]]
    assert W[8 * r + i, n] == 9.0                         # group 0: s = 1
    # same code in group 1 (rows 128..255) picks up s = 1/2
    qw2 = np.zeros_like(qw)
    qw2[16 + r, n] = np.uint32(9) << np.uint32(4 * i)
    W2 = oracle.dequant_gptq(qw2.view(np.int32), s, qz.view(np.int32))
    assert np.argwhere(W2 != 0).tolist() == [[128 + 8 * r + i, n]]
    assert W2[128 + 8 * r + i, n] == 4.5


def test_dequant_zero_nibble_order():
    K, N = 128, 16
    qw = np.zeros((K // 8, N), np.uint32)
    qz = np.zeros((1, N // 8), np.uint32)
    qz[0, 1] = np.uint32(3) << np.uint32(4 * 5)           # zero of column 8+5
    s = np.ones((1, N), np.float16)
    W = oracle.dequant_gptq(qw.view(np.int32), s, qz.view(np.int32))
    assert np.all(W[:, 13] == -3.0)
    W[:, 13] = 0
    assert np.all(W == 0)


def test_unpack_all_code_zero_pairs():
    # every (q, z) pair in 0..15 x 0..15 survives pack -> unpack
    K, N = 128, 256
    q = np.zeros((K, N), np.uint8)
    z = np.zeros((1, N), np.uint8)
    for n in range(N):
        q[:, n] = n % 16
        z[0, n] = n // 16
    qw = np.zeros((K // 8, N), np.uint32)
    for r in range(K // 8):
        for n in range(N):
            qw[r, n] = _pack_words(q[8 * r:8 * r + 8, n])
    qz = np.zeros((1, N // 8), np.uint32)
    for c in range(N // 8):
        qz[0, c] = _pack_words(z[0, 8 * c:8 * c + 8])
    uq, uz = oracle.unpack_gptq(qw.view(np.int32), qz.view(np.int32))
    assert np.array_equal(uq, q) and np.array_equal(uz, z)
    W = oracle.dequant_gptq(qw.view(np.int32), np.ones((1, N), np.float16), qz.view(np.int32))
    assert np.array_equal(W[0], (np.arange(N) % 16) - (np.arange(N) // 16))


def test_golden_dequant_fixture():
    with open(os.path.join(GOLDEN, "gptq_dequant_closed_form.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        K, N = 128, 8
        qw = np.zeros((K // 8, N), np.uint32)
        qw[0, 0] = np.uint32(int(case["qword"], 16))
        qz = np.zeros((1, 1), np.uint32)
        qz[0, 0] = np.uint32(int(case["zword"], 16))
        s = np.full((1, N), case["scale"], np.float16)
        W = oracle.dequant_gptq(qw.view(np.int32), s, qz.view(np.int32))
        assert W[:8, 0].tolist() == case["expected_rows0to7_col0"]


def test_rtn_quantizer_error_bound():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float16)
    qw, s, qz = synth.gptq_from_linear(w)               # [N,K] -> GPTQ [K,N]
    W = oracle.dequant_gptq(qw, s, qz)
    sg = np.repeat(s.astype(np.float64), 128, axis=0)
    err = np.abs(W - w.T.astype(np.float64))
    assert np.all(err <= 0.51 * sg)


# ------------------------------------------------------------------ FFN ----

def _int4_expert(w13, w2):
    return synth.expert_int4(w13, w2)


def test_zero_codes_give_zero_output():
    H, I = 256, 128
    m13 = _mat(H, 2 * I, 7, 7, 0.5)
    m2 = _mat(I, H, 7, 7, 0.5)
    x = np.random.default_rng(0).standard_normal((3, H)).astype(np.float16)
    y = oracle.expert_ffn_int4(x, m13, m2)
    assert np.all(y == 0)


def test_swiglu_closed_form_one_hot():
    # x = e_0.  gate column 0 of W13 = a, up = b, W2 = identity block:
    # y[n] = silu(a_n) * b_n with silu(ln 3) = 0.75 ln 3, silu(0) = 0,
    # silu(-ln 3) = -0.25 ln 3.  Swapping gate and up would give silu(b)*a.
    H = I = 128
    l3 = float(np.float16(np.log(3.0)))
    a = np.zeros(I)
    b = np.zeros(I)
    a[:3] = [l3, 0.0, -l3]
    b[:3] = [2.0, 5.0, 4.0]
    w13 = np.zeros((2 * I, H), np.float16)
    w13[:I, 0] = a
    w13[I:, 0] = b
    w2 = np.eye(H, I, dtype=np.float16)
    x = np.zeros((1, H), np.float16)
    x[0, 0] = 1.0
    y = oracle.expert_ffn_f16(x, w13, w2)[0]
    sig = lambda v: 1.0 / (1.0 + np.exp(-v))
    exp = [l3 * sig(l3) * 2.0, 0.0, -l3 * sig(-l3) * 4.0]
    assert np.allclose(y[:3], exp, rtol=1e-14, atol=0)
    assert abs(y[0] - 1.5 * np.log(3.0)) < 2e-3           # 0.75 ln3 * 2
    assert np.all(y[3:] == 0)


def _tiny_layer(seed=0, E=6, H=256, I=128):
    rng = np.random.default_rng(seed)
    f16 = []
    for _ in range(E):
        w13 = (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float16)
        w2 = (rng.standard_normal((H, I)) * 0.02).astype(np.float16)
        f16.append((w13, w2))
    q = [_int4_expert(*p) for p in f16]
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float16)
    return f16, q, wr


@pytest.mark.parametrize("kind", ["f16", "int4"])
def test_grouped_equals_masked_brute_force(kind):
    f16, q, wr = _tiny_layer(1)
    E, k, T = 6, 2, 7
    x = np.random.default_rng(9).standard_normal((T, 256)).astype(np.float16)
    r = oracle.route_topk(x, wr, k)
    m = oracle.gather_maps(r["ids"], E)
    experts = f16 if kind == "f16" else q
    y = oracle.grouped_ffn(x, m, experts, kind)
    # every expert on every token, then select
    allout = np.stack([
        (oracle.expert_ffn_f16(x, *f16[e]) if kind == "f16"
         else oracle.expert_ffn_int4(x, q[e]["w13"], q[e]["w2"])) for e in range(E)])
    for p in range(T * k):
        t, e = p // k, int(r["ids"].ravel()[p])
        assert np.allclose(y[m["pair_pos"][p]], allout[e, t], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("kind", ["f16", "int4"])
def test_grouped_equals_per_token_gemv(kind):
    f16, q, wr = _tiny_layer(2)
    E, k, T = 6, 3, 9
    x = np.random.default_rng(4).standard_normal((T, 256)).astype(np.float16)
    r = oracle.route_topk(x, wr, k)
    m = oracle.gather_maps(r["ids"], E)
    experts = f16 if kind == "f16" else q
    y = oracle.grouped_ffn(x, m, experts, kind)
    pt = oracle.per_token_ffn(x, r["ids"], experts, kind)
    for t in range(T):
        for j in range(k):
            a = y[m["pair_pos"][t * k + j]]
            assert np.max(np.abs(a - pt[t, j])) <= 1e-12 * max(1.0, np.max(np.abs(pt[t, j])))


def test_fp32_oracle_close_to_fp64():
    f16, q, wr = _tiny_layer(3)
    x = np.random.default_rng(5).standard_normal((5, 256)).astype(np.float16)
    for kind, ex in (("f16", f16), ("int4", q)):
        a = oracle.moe_layer(x, wr, 2, ex, kind, dtype=np.float64)["out"]
        b = oracle.moe_layer(x, wr, 2, ex, kind, dtype=np.float32)["out"]
        assert np.linalg.norm(a - b) / np.linalg.norm(a) <= 1e-6


def test_int4_dequant_is_exact_in_fp32():
    f16, q, _ = _tiny_layer(4)
    a = oracle.dequant_gptq(*q[0]["w13"], dtype=np.float32).astype(np.float64)
    b = oracle.dequant_gptq(*q[0]["w13"], dtype=np.float64)
    assert np.array_equal(a, b)


def test_two_shared_experts_equal_one_concatenated():
    sh = synth.shared_expert(synth.DS)
    x = synth.tokens(synth.DS, 2)
    (a13, a2), (b13, b2) = sh["parts"]
    two = oracle.expert_ffn_f16(x, a13, a2) + oracle.expert_ffn_f16(x, b13, b2)
    one = oracle.expert_ffn_f16(x, sh["w13"], sh["w2"])
    assert np.max(np.abs(two - one)) <= 1e-12


def test_single_expert_layer_is_dense_mlp():
    # E = 1, k = 1, renormalised: the MoE layer is exactly that expert.
    f16, q, _ = _tiny_layer(6, E=1)
    wr = np.zeros((1, 256), np.float16)
    x = np.random.default_rng(7).standard_normal((4, 256)).astype(np.float16)
    out = oracle.moe_layer(x, wr, 1, f16, "f16", renormalize=True)
    assert np.all(out["route"]["weights"] == 1.0)
    assert np.array_equal(out["out"], oracle.expert_ffn_f16(x, *f16[0]))


# -------------------------------------------------------------- combine ----

def test_combine_k1_identity():
    y = np.random.default_rng(0).standard_normal((5, 64)).astype(np.float16)
    pp = np.array([3, 0, 4, 1, 2])
    out = oracle.combine(y, pp, np.ones((5, 1)))
    assert np.array_equal(oracle.to_f16(out), y[pp])


def test_combine_hand_sums():
    # rows hold constants; t=0 takes rows 0 (w .25) and 2 (w .5);
    # t=1 rows 1 (w 1) and 3 (w .125); shared 4 and 8 with scale .5 / 1
    y = np.array([[1.0] * 4, [2.0] * 4, [3.0] * 4, [8.0] * 4])
    pp = np.array([0, 2, 1, 3])
    w = np.array([[0.25, 0.5], [1.0, 0.125]])
    sh = np.array([[4.0] * 4, [8.0] * 4])
    out = oracle.combine(y, pp, w, sh, np.array([0.5, 1.0]))
    assert out[0].tolist() == [3.75] * 4          # .25 + 1.5 + 2
    assert out[1].tolist() == [11.0] * 4          # 2 + 1 + 8
    res = oracle.combine(y, pp, w, None, None, residual=np.array([[1.0] * 4, [2.0] * 4]))
    assert res[0].tolist() == [2.75] * 4 and res[1].tolist() == [5.0] * 4


def test_combine_skips_dropped_pairs():
    y = np.ones((1, 4))
    out = oracle.combine(y, np.array([0, -1]), np.array([[0.5, 0.5]]))
    assert out[0].tolist() == [0.5] * 4


# ------------------------------------------------------------ generator ----

def test_generator_deterministic():
    import hashlib
    h = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    a = synth.make_layer(synth.TINY, experts=[0, 3])
    b = synth.make_layer(synth.TINY, experts=[0, 3])
    assert h(a["router"]) == h(b["router"])
    for e in (0, 3):
        assert h(a["f16"][e][0]) == h(b["f16"][e][0])
        assert h(a["int4"][e]["w13"][0]) == h(b["int4"][e]["w13"][0])
    assert h(synth.tokens(synth.TINY, 4, step=1)) != h(synth.tokens(synth.TINY, 4, step=2))
    w = a["f16"][0][0].astype(np.float64)
    assert abs(w.std() - 0.02) < 0.002 and abs(w.mean()) < 0.002


def test_torch_rtn_matches_numpy_rtn():
    # the device-side generator's quantiser is the same RTN rule (run on CPU)
    import torch
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float16)
    a = synth.gptq_from_linear(w)
    b = synth.torch_gptq_from_linear(torch.from_numpy(w))
    for x, y in zip(a, b):
        assert np.array_equal(x, y.numpy())


def test_rms_norm_closed_forms():
    x = np.array([[3.0] * 8, [-2.0] * 8, [1.0, -1.0] * 4])
    y = oracle.rms_norm(x, eps=0.0)
    assert np.allclose(y, np.sign(x), rtol=0, atol=1e-15)
    z = oracle.rms_norm(np.zeros((1, 4)), eps=1e-6)
    assert np.all(z == 0)
    rng = np.random.default_rng(2)
    a = rng.standard_normal((5, 256))
    assert np.allclose(oracle.rms_norm(a * 7.0, eps=0.0), oracle.rms_norm(a, eps=0.0))
    assert np.allclose(np.mean(oracle.rms_norm(a, eps=0.0) ** 2, axis=1), 1.0)
    # eps sits inside the root, added to the mean square: sqrt(1 + 3) = 2
    assert np.allclose(oracle.rms_norm(np.ones((1, 4)), eps=3.0), 0.5, rtol=0, atol=1e-15)


def test_moe_layer_residual_is_added_once():
    """Zero expert weights: the pre-norm block returns its residual input
    exactly (rounded to fp16), whichever way the residual is passed."""
    s = synth.TINY
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, s.H)).astype(np.float16)
    res = rng.standard_normal((3, s.H)).astype(np.float16)
    zero = [(np.zeros((2 * s.I, s.H), np.float16), np.zeros((s.H, s.I), np.float16))] * s.E
    wr = synth.router(s)
    out = oracle.moe_layer(x, wr, s.k, zero, "f16", residual=res)["out"]
    assert np.array_equal(out, res)
    out = oracle.moe_layer(x, wr, s.k, zero, "f16", residual=True)["out"]
    assert np.array_equal(out, x)
    out = oracle.moe_layer(x, wr, s.k, zero, "f16")["out"]
    assert np.array_equal(out, np.zeros_like(x))
