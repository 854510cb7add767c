"""Pins for the oracle's INT4 draft expert and the shared-expert wiring of a
layer, against values fixed by hand rather than by another oracle call.

* Weights placed exactly on the quantisation grid (w = (q - z) * s with a
  power-of-two s per group and column) are representable in fp16, so the
  INT4 draft expert built from their codes must equal the FP16 target expert
  on the same weights ("Specter previews expert routing with an INT4 copy of
  the model itself", What shipped: the draft's routed experts are a GPTQ INT4
  group-128 copy of the target's).  The codes are packed here by hand, not by
  the input generator.
* A one-hot token through hand-packed INT4 codes gives silu(a) * b at
  hand-picked output columns, with silu(1) = e / (1 + e) written out as
  decimals: a gate/up swap, a transposed down projection or a wrong nibble
  order each move or change them.
* A layer whose routed experts are all zero returns sigmoid(x . w_sg) times
  the shared expert's output ("Specter: Fast MoE Inference via
  Quantization-Enabled Multi-Step Speculative Offloading", Key Contributions
  2: gating and shared experts stay FP16), with sigmoid(2) written out.
"""
import numpy as np
import pytest

import oracle

GROUP = 128

# silu(v) = v / (1 + e^-v) evaluated by hand at the points used below
SILU_1 = 0.7310585786300049          # e / (1 + e)
SILU_M1 = -0.2689414213699951        # -1 / (1 + e)
SILU_HALF = 0.3112296656009273       # 0.5 / (1 + e^-0.5)
SIGMOID_2 = 0.8807970779778823       # 1 / (1 + e^-2)


def _pack_codes(q_kn, z_gn, s_gn):
    """Hand GPTQ packing of codes q [K, N] (0..15), zeros z [K/128, N] and
    scales s [K/128, N]: nibble i of qweight[r, n] is row 8r+i; nibble i of
    qzeros[g, c] is column 8c+i."""
    K, N = q_kn.shape
    qw = np.zeros((K // 8, N), np.uint64)
    for i in range(8):
        qw |= q_kn[i::8, :].astype(np.uint64) << np.uint64(4 * i)
    G = K // GROUP
    qz = np.zeros((G, N // 8), np.uint64)
    for i in range(8):
        qz |= z_gn[:, i::8].astype(np.uint64) << np.uint64(4 * i)
    return (qw.astype(np.uint32).view(np.int32), s_gn.astype(np.float16),
            qz.astype(np.uint32).view(np.int32))


def _grid_matrix(rng, K, N):
    """Random codes, zeros and power-of-two scales; returns the packed matrix
    and its exact weights w [K, N] = (q - z) * s (fp16-exact)."""
    q = rng.integers(0, 16, size=(K, N)).astype(np.uint8)
    z = rng.integers(0, 16, size=(K // GROUP, N)).astype(np.uint8)
    s = (2.0 ** -rng.integers(5, 9, size=(K // GROUP, N))).astype(np.float64)
    g = np.arange(K) // GROUP
    w = (q.astype(np.float64) - z[g, :]) * s[g, :]
    assert np.array_equal(w.astype(np.float16).astype(np.float64), w)   # exact in fp16
    return _pack_codes(q, z, s), w


@pytest.mark.parametrize("H,I,T", [(256, 128, 3), (384, 256, 5)])
def test_int4_expert_equals_f16_expert_on_the_grid(H, I, T):
    rng = np.random.default_rng(H + I)
    m13, w13_kn = _grid_matrix(rng, H, 2 * I)     # w13^T [H, 2I]: gate columns first
    m2, w2_kn = _grid_matrix(rng, I, H)           # w2^T [I, H]
    w13 = w13_kn.T.astype(np.float16)             # nn.Linear [2I, H]
    w2 = w2_kn.T.astype(np.float16)               # nn.Linear [H, I]
    x = rng.standard_normal((T, H)).astype(np.float16)
    a = oracle.expert_ffn_int4(x, m13, m2)
    b = oracle.expert_ffn_f16(x, w13, w2)
    assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))
    # and the same through the grouped loop of a layer with these experts
    ids = np.zeros((T, 1), np.int32)
    maps = oracle.gather_maps(ids, 1)
    ya = oracle.grouped_ffn(x, maps, [dict(w13=m13, w2=m2)], "int4")
    yb = oracle.grouped_ffn(x, maps, [(w13, w2)], "f16")
    assert np.max(np.abs(ya - yb)) <= 1e-12 * max(1.0, np.max(np.abs(yb)))


def _one_hot_int4_expert(H=256, I=128):
    """Codes for: gate column n (row 0) = a_n, up column n (row 0) = b_n,
    every other weight of w13 zero; W2[i, H-1-i] = 1 for i < 4, else zero.
    Scales 1/2 for w13 and 1 for w2, zeros 8 (a code equal to its zero is a
    zero weight)."""
    a = [1.0, 0.0, -1.0, 0.5]
    b = [2.0, 3.0, 4.0, -1.0]
    q13 = np.full((H, 2 * I), 8, np.uint8)
    z13 = np.full((H // GROUP, 2 * I), 8, np.uint8)
    s13 = np.full((H // GROUP, 2 * I), 0.5)
    for n in range(4):
        q13[0, n] = 8 + int(a[n] / 0.5)
        if b[n] == 4.0:                    # q - z = 8 needs z = 7, q = 15
            z13[0, I + n] = 7
            q13[1:GROUP, I + n] = 7
            q13[0, I + n] = 15
        else:
            q13[0, I + n] = 8 + int(b[n] / 0.5)
    q2 = np.full((I, H), 8, np.uint8)
    z2 = np.full((I // GROUP, H), 8, np.uint8)
    s2 = np.ones((I // GROUP, H))
    for i in range(4):
        q2[i, H - 1 - i] = 9
    return _pack_codes(q13, z13, s13), _pack_codes(q2, z2, s2)


def test_int4_expert_one_hot_closed_form():
    H, I = 256, 128
    m13, m2 = _one_hot_int4_expert(H, I)
    x = np.zeros((1, H), np.float16)
    x[0, 0] = 1.0
    y = oracle.expert_ffn_int4(x, m13, m2)[0]
    expect = np.zeros(H)
    expect[H - 1] = SILU_1 * 2.0          # 1.4621171572600098
    expect[H - 2] = 0.0                   # silu(0) * 3
    expect[H - 3] = SILU_M1 * 4.0         # -1.0757656854799804
    expect[H - 4] = SILU_HALF * -1.0      # -0.3112296656009273
    assert np.allclose(y, expect, rtol=1e-14, atol=1e-15)


def _one_hot_shared(H=256, Is=128):
    """FP16 shared expert: gate row 0 = e_0, up row 0 = 2 e_0, w2[3, 0] = 1,
    so FFN_shared(e_0) = silu(1) * 2 at column 3 and zero elsewhere."""
    w13 = np.zeros((2 * Is, H), np.float16)
    w13[0, 0] = 1.0
    w13[Is, 0] = 2.0
    w2 = np.zeros((H, Is), np.float16)
    w2[3, 0] = 1.0
    return w13, w2


@pytest.mark.parametrize("kind", ["f16", "int4"])
def test_layer_with_zero_routed_experts_is_gated_shared_expert(kind):
    H, I, E, k = 256, 128, 6, 2
    rng = np.random.default_rng(12)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float16)
    if kind == "f16":
        routed = [(np.zeros((2 * I, H), np.float16), np.zeros((H, I), np.float16))] * E
    else:
        zero = np.full((H, 2 * I), 3, np.uint8)
        z13 = np.full((H // GROUP, 2 * I), 3, np.uint8)
        zero2 = np.full((I, H), 3, np.uint8)
        z2 = np.full((I // GROUP, H), 3, np.uint8)
        routed = [dict(w13=_pack_codes(zero, z13, np.ones((H // GROUP, 2 * I))),
                       w2=_pack_codes(zero2, z2, np.ones((I // GROUP, H))))] * E
    w13s, w2s = _one_hot_shared(H)
    x = np.zeros((1, H), np.float16)
    x[0, 0] = 1.0
    gate = np.zeros(H, np.float16)
    gate[0] = 2.0                         # x . w_sg = 2
    out = oracle.moe_layer(x, wr, k, routed, kind,
                           shared=dict(w13=w13s, w2=w2s, gate=gate))["out"][0]
    expect = np.zeros(H)
    expect[3] = SIGMOID_2 * SILU_1 * 2.0  # 1.2878285197759445
    assert np.allclose(out, expect, rtol=1e-14, atol=1e-15)
    # without a gate vector (DeepSeek-style shared experts) the term is unscaled
    out = oracle.moe_layer(x, wr, k, routed, kind, shared=dict(w13=w13s, w2=w2s))["out"][0]
    expect[3] = SILU_1 * 2.0
    assert np.allclose(out, expect, rtol=1e-14, atol=1e-15)
    # the residual adds once on top of the gated shared term
    res = np.zeros((1, H), np.float16)
    res[0, 3] = 1.0
    out = oracle.moe_layer(x, wr, k, routed, kind, shared=dict(w13=w13s, w2=w2s, gate=gate),
                           residual=res)["out"][0]
    assert np.isclose(out[3], 1.0 + SIGMOID_2 * SILU_1 * 2.0, rtol=1e-14, atol=0)


def test_layer_routed_plus_gated_shared_closed_form():
    """Routed and shared terms together: one routed expert (E = 1, k = 1,
    renormalised so its weight is exactly 1) computing silu(1)*2 at column
    H-1, plus the gated shared expert at column 3."""
    H, I = 256, 128
    m13, m2 = _one_hot_int4_expert(H, I)
    wr = np.zeros((1, H), np.float16)
    w13s, w2s = _one_hot_shared(H)
    gate = np.zeros(H, np.float16)
    gate[0] = 2.0
    x = np.zeros((1, H), np.float16)
    x[0, 0] = 1.0
    out = oracle.moe_layer(x, wr, 1, [dict(w13=m13, w2=m2)], "int4",
                           shared=dict(w13=w13s, w2=w2s, gate=gate), renormalize=True)
    y = out["out"][0]
    assert np.isclose(y[H - 1], SILU_1 * 2.0, rtol=1e-14, atol=0)
    assert np.isclose(y[H - 3], SILU_M1 * 4.0, rtol=1e-14, atol=0)
    assert np.isclose(y[3], SIGMOID_2 * SILU_1 * 2.0, rtol=1e-14, atol=0)
    assert np.isclose(out["route"]["gate"][0], SIGMOID_2, rtol=1e-15, atol=0)


# silu at the points the AWQ one-hot case reaches, written out
SILU_Q = 0.14054412522144952         # 0.25 / (1 + e^-0.25)
SILU_MHALF = -0.1887703343990727     # -0.5 / (1 + e^0.5)


def test_awq_unit_factors_equal_gptq_expert():
    rng = np.random.default_rng(41)
    H, I = 256, 128
    m13, _ = _grid_matrix(rng, H, 2 * I)
    m2, _ = _grid_matrix(rng, I, H)
    x = rng.standard_normal((3, H)).astype(np.float16)
    a = oracle.expert_ffn_awq(x, m13, m2, np.ones(H, np.float16), np.ones(I, np.float16))
    b = oracle.expert_ffn_int4(x, m13, m2)
    assert np.array_equal(a, b)


def test_awq_one_hot_closed_form():
    """The one-hot INT4 expert above with factor 2 on hidden channel 0 and 4
    on intermediate channel 0: g = a/2, u = b/2, h = silu(g) u, and h_0 / 4
    reaches output column H-1."""
    H, I = 256, 128
    m13, m2 = _one_hot_int4_expert(H, I)
    a13 = np.full(H, 3.0, np.float16)
    a13[0] = 2.0
    a2 = np.ones(I, np.float16)
    a2[0] = 4.0
    x = np.zeros((1, H), np.float16)
    x[0, 0] = 1.0
    y = oracle.expert_ffn_awq(x, m13, m2, a13, a2)[0]
    expect = np.zeros(H)
    expect[H - 1] = SILU_HALF * 1.0 / 4.0      # g = 1/2, u = 2/2;  0.07780741640023182
    expect[H - 2] = 0.0                         # silu(0) * 3/2
    expect[H - 3] = SILU_MHALF * 2.0            # g = -1/2, u = 4/2; -0.3775406687981454
    expect[H - 4] = SILU_Q * -0.5               # g = 1/4, u = -1/2; -0.07027206261072476
    assert np.allclose(y, expect, rtol=1e-14, atol=1e-15)


def test_awq_generator_approximates_target():
    """The AWQ-style draft of a target expert: its codes are the RTN
    quantisation of the input-channel-scaled weights (error within half a
    step), and through the expert it still approximates the FP16 expert at
    4-bit accuracy.  Random factors make it somewhat less accurate than the
    plain GPTQ draft (scaled-up channels widen their groups' ranges); AWQ's
    own factors come from activation statistics, which need data."""
    import synth
    s = synth.TINY
    w13, w2 = synth.expert_f16(s, 0, 1)
    ex = synth.expert_awq(s, 0, 1, w13, w2)
    assert ex["a13"].shape == (s.H,) and ex["a2"].shape == (s.I,)
    assert np.all(ex["a13"] >= 0.5) and np.all(ex["a13"] <= 2.0)
    W = oracle.dequant_gptq(*ex["w13"])                        # [H, 2I]
    scaled = w13.T.astype(np.float64) * ex["a13"].astype(np.float64)[:, None]
    step = np.repeat(ex["w13"][1].astype(np.float64), 128, axis=0)
    assert np.all(np.abs(W - scaled) <= 0.51 * step + 1e-3 * np.abs(scaled))
    x = synth.tokens(s, 4, step=3)
    ref = oracle.expert_ffn_f16(x, w13, w2)
    a = oracle.expert_ffn_awq(x, ex["w13"], ex["w2"], ex["a13"], ex["a2"])
    g = synth.expert_int4(w13, w2)
    b = oracle.expert_ffn_int4(x, g["w13"], g["w2"])
    ea = np.linalg.norm(a - ref) / np.linalg.norm(ref)
    eb = np.linalg.norm(b - ref) / np.linalg.norm(ref)
    assert ea < 0.5 and eb < 0.5 and ea < 2.5 * eb
