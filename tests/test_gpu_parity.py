"""GPU parity: every entry point of libsmoe.so against the CPU oracle on the
same seeded inputs.  Integer outputs (ids, counters, maps) must match exactly;
FP16 outputs within normalised L2 5e-3 and max |err| 2e-2; routing weights
within 1e-5 relative."""
import dataclasses

import numpy as np
import pytest
import torch

import fp16_verify_expert_amd as fve
import oracle
import synth
from gpu_util import (W_RTOL, Layer, assert_fp16_close, dev, host, run_layer, say, upload_f16,
                      upload_int4)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    fve.lib()
    torch.cuda.init()


def _err():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


# ---------------------------------------------------------------- S1 ----

# the ABI's largest routers: 256 experts, top-32 (the fused draft step's limit)
_E256 = dataclasses.replace(synth.TINY, name="tiny_e256_k32", E=256, k=32)
ROUTE_CASES = [(synth.TINY, 4), (synth.TINY, 1), (synth.DS, 1), (synth.DS, 16), (synth.QWEN, 9),
               (synth.QWEN, 17), (synth.PHI, 1), (synth.PHI, 17), (synth.DS, 257), (_E256, 1),
               (_E256, 5)]


@pytest.mark.parametrize("shape,T", ROUTE_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_route_topk(shape, T):
    say(f"route {shape.name} T={T}")
    wr = synth.router(shape)
    x = synth.tokens(shape, T, step=3)
    sh = synth.shared_expert(shape)
    gvec = None if sh is None else sh.get("gate")
    ref = oracle.route_topk(x, wr, shape.k, shape.renormalize, gvec)
    ids, w, gate = fve.moe_route_topk(dev(x), dev(wr), shape.k, shape.renormalize,
                                      None if gvec is None else dev(gvec))
    assert np.array_equal(host(ids), ref["ids"])
    assert np.allclose(host(w), ref["weights"], rtol=W_RTOL, atol=1e-7)
    if gvec is not None:
        assert np.allclose(host(gate), ref["gate"], rtol=W_RTOL, atol=1e-7)


def test_route_nan_logits_rank_last():
    # NaN logits rank below every number (the oracle's sort puts them last);
    # the ids stay valid and distinct
    s = synth.TINY
    x = synth.tokens(s, 2)
    w = synth.router(s).copy()
    w[3, 0] = np.float16(np.inf)       # inf * 0-crossing products give NaN for x[0]=... below
    x[:, 0] = 0.0                      # 0 * inf = NaN in expert 3's logit
    ids, _, _ = fve.moe_route_topk(dev(x), dev(w), s.E)
    ref = oracle.route_topk(x, w, s.E)
    assert np.isnan(ref["logits32"][:, 3]).all()
    assert np.array_equal(host(ids), ref["ids"])
    assert host(ids)[:, -1].tolist() == [3, 3]


def test_route_renormalize_and_ties():
    s = synth.TINY
    wr = synth.router(s)
    x = np.zeros((3, s.H), np.float16)
    ids, w, _ = fve.moe_route_topk(dev(x), dev(wr), 3)
    assert host(ids).tolist() == [[0, 1, 2]] * 3
    assert np.allclose(host(w), 1.0 / s.E, rtol=1e-6)
    x = synth.tokens(s, 5)
    ref = oracle.route_topk(x, wr, 3, renormalize=True)
    ids, w, _ = fve.moe_route_topk(dev(x), dev(wr), 3, True)
    assert np.array_equal(host(ids), ref["ids"])
    assert np.allclose(host(w), ref["weights"], rtol=W_RTOL)
    # k == E: the full ranking
    ref = oracle.route_topk(x, wr, s.E)
    ids, w, _ = fve.moe_route_topk(dev(x), dev(wr), s.E)
    assert np.array_equal(host(ids), ref["ids"])


def test_route_pinned_order_cases():
    # the hand cases of the oracle pins, through the kernel: 2^24 + ones
    for H, ones, want in ((512, range(1, 8), 2.0 ** 24), (1024, (512, 513), 2.0 ** 24),
                          (512, (8, 24), 2.0 ** 24 + 2)):
        x = np.zeros((1, H), np.float16)
        w = np.zeros((2, H), np.float16)
        x[0, 0] = w[0, 0] = 4096.0
        for h in ones:
            x[0, h] = w[0, h] = 1.0
        w[1, 0] = 4096.0            # expert 1 logit: exactly 2^24
        ids, wt, _ = fve.moe_route_topk(dev(x), dev(w), 2)
        # expert 0 wins iff its logit rounds above 2^24; equal -> lower id
        assert host(ids)[0].tolist() == [0, 1]
        p0 = host(wt)[0, 0]
        expect = 1.0 / (1.0 + np.exp(2.0 ** 24 - want))
        assert abs(p0 - expect) < 1e-6


# ---------------------------------------------------------------- S2 ----

def test_elb_count_accumulates():
    s = synth.QWEN_CHUNK
    wr = synth.router(s)
    L = 24
    counters = torch.zeros((L, s.E), dtype=torch.int32, device="cuda")
    ref = np.zeros((L, s.E), np.int32)
    err = _err()
    for step in range(16):
        for layer in (0, 5, 23):
            x = synth.tokens(s, 1, step=step, layer=layer)
            r = oracle.route_topk(x, wr, s.k)
            ids, _, _ = fve.moe_route_topk(dev(x), dev(wr), s.k)
            fve.elb_count(ids, s.E, layer, counters, err)
            ref = oracle.elb_update(ref, r["ids"], layer)
    c = host(counters)
    assert np.array_equal(c, ref)
    assert c[0].sum() == 16 * s.k and c[1].sum() == 0
    assert int(host(err)[0]) == 0


def test_elb_count_bad_ids_flagged():
    ids = dev(np.array([[0, 7], [8, -1], [3, 3]], np.int32))
    counters = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    err = _err()
    fve.elb_count(ids, 8, 1, counters, err)
    assert host(counters)[1].tolist() == [1, 0, 0, 2, 0, 0, 0, 1]
    assert int(host(err)[0]) & fve.SMOE_DERR_BAD_ID


# ---------------------------------------------------------------- S3 ----

# up to 1024 pairs the ids are sorted in LDS by one kernel, above by chunks
GATHER_CASES = [(4, 2, 8), (1, 6, 64), (16, 6, 64), (17, 4, 60), (9, 4, 60), (17, 2, 16),
                (300, 8, 64), (2000, 2, 16), (1, 1, 1), (5, 256, 256), (128, 8, 64),
                (512, 2, 16)]


@pytest.mark.parametrize("T,k,E", GATHER_CASES)
def test_gather_maps(T, k, E):
    rng = np.random.default_rng(T * 1000 + k * 10 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if T in (2000, 512):  # heavily skewed: most pairs on two experts
        ids[:, 0] = rng.integers(0, 2, size=T)
        ids[:, 1] = np.where(ids[:, 0] == 0, 1, 0)
    ref = oracle.gather_maps(ids, E)
    m = fve.moe_gather(dev(ids), E, _err())
    n = T * k
    for key in ("offsets", "active"):
        assert np.array_equal(host(m[key]), ref[key]), key
    for key in ("sorted_token", "sorted_pair", "pair_pos"):
        assert np.array_equal(host(m[key])[:n], ref[key]), key
    assert int(host(m["n_active"])[0]) == int(ref["n_active"])


def test_gather_bad_ids_and_empty():
    ids = np.array([[1, 9], [0, -3], [1, 2]], np.int32)
    err = _err()
    m = fve.moe_gather(dev(ids), 4, err)
    ref = oracle.gather_maps(ids, 4)
    assert host(m["offsets"]).tolist() == ref["offsets"].tolist()
    assert host(m["pair_pos"]).tolist() == ref["pair_pos"].tolist()
    assert host(m["sorted_pair"]).tolist() == ref["sorted_pair"].tolist()
    assert int(host(err)[0]) & fve.SMOE_DERR_BAD_ID
    m = fve.moe_gather(torch.zeros((0, 2), dtype=torch.int32, device="cuda"), 4)
    assert host(m["offsets"]).tolist() == [0] * 5
    assert int(host(m["n_active"])[0]) == 0
    assert host(m["active"]).tolist() == [-1] * 4


# ------------------------------------------------ S1 + S2 + S3 fused ----

PLAN_CASES = [(synth.TINY, 1), (synth.TINY, 37), (synth.TINY, 455), (synth.DS, 1),
              (synth.DS, 16), (synth.DS, 62), (synth.QWEN, 1), (synth.QWEN, 17), (synth.PHI, 1),
              (synth.PHI, 17), (_E256, 1), (_E256, 3)]


@pytest.mark.parametrize("spread", [True, False], ids=["logits_ws", "no_ws"])
@pytest.mark.parametrize("shape,T", PLAN_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_route_plan_matches_separate_calls(shape, T, spread):
    """The fused plan equals routing + ELB + gather bit for bit, and the oracle,
    with a logits workspace (steps with T*(E+1)*H above 2^16 spread their dot
    products over the chip; the workspace starts as NaN so nothing depends on
    its contents) and without one."""
    say(f"route plan {shape.name} T={T} spread={spread}")
    E, k = shape.E, shape.k
    wr = synth.router(shape)
    x = synth.tokens(shape, T, step=5)
    sh = synth.shared_expert(shape)
    gvec = None if sh is None else sh.get("gate")
    dgvec = None if gvec is None else dev(gvec)
    c0 = np.random.default_rng(T).integers(0, 50, size=(3, E)).astype(np.int32)
    counters = dev(c0)
    err = _err()
    lws = None
    if spread:
        lws = torch.full((T * (E + 1),), float("nan"), dtype=torch.float32, device="cuda")
    ids, w, gate, m = fve.moe_route_plan(dev(x), dev(wr), k, shape.renormalize, dgvec,
                                         counters=counters, layer=1, err_word=err,
                                         logits_ws=lws, spread=spread)
    ids2, w2, gate2 = fve.moe_route_topk(dev(x), dev(wr), k, shape.renormalize, dgvec)
    counters2 = dev(c0)
    fve.elb_count(ids2, E, 1, counters2)
    m2 = fve.moe_gather(ids2, E)
    n = T * k
    assert torch.equal(ids, ids2)
    assert torch.equal(w, w2)
    if gvec is not None:
        assert torch.equal(gate, gate2)
    assert torch.equal(counters, counters2)
    for key in ("offsets", "active", "n_active"):
        assert torch.equal(m[key], m2[key]), key
    for key in ("sorted_token", "sorted_pair", "pair_pos"):
        assert torch.equal(m[key][:n], m2[key][:n]), key
    ref = oracle.route_topk(x, wr, k, shape.renormalize, gvec)
    assert np.array_equal(host(ids), ref["ids"])
    assert np.array_equal(host(counters), oracle.elb_update(c0, ref["ids"], 1))
    rm = oracle.gather_maps(ref["ids"], E)
    assert np.array_equal(host(m["offsets"]), rm["offsets"])
    assert np.array_equal(host(m["sorted_pair"])[:n], rm["sorted_pair"])
    assert int(host(err)[0]) == 0


def test_route_plan_empty_and_no_counters():
    s = synth.TINY
    wr = dev(synth.router(s))
    _, _, _, m = fve.moe_route_plan(torch.zeros((0, s.H), dtype=torch.float16, device="cuda"),
                                    wr, s.k)
    assert host(m["offsets"]).tolist() == [0] * (s.E + 1)
    assert int(host(m["n_active"])[0]) == 0
    assert host(m["active"]).tolist() == [-1] * s.E
    x = synth.tokens(s, 3, step=2)
    ids, _, _, m = fve.moe_route_plan(dev(x), wr, s.k)
    ref = oracle.route_topk(x, synth.router(s), s.k)
    assert np.array_equal(host(ids), ref["ids"])
    # the two-launch forms (spread logits, or the routing kernel when no
    # workspace is given) without counters: the same maps as moe_gather on the
    # same ids
    xd = synth.tokens(synth.DS, 16, step=5)
    wd = dev(synth.router(synth.DS))
    for spread in (True, False):
        ids2, _, _, m2 = fve.moe_route_plan(dev(xd), wd, synth.DS.k, spread=spread)
        g2 = fve.moe_gather(ids2, synth.DS.E)
        torch.cuda.synchronize()
        assert np.array_equal(host(ids2), oracle.route_topk(xd, synth.router(synth.DS),
                                                            synth.DS.k)["ids"])
        for key in ("offsets", "active", "n_active", "sorted_token", "sorted_pair", "pair_pos"):
            assert torch.equal(m2[key], g2[key]), key
    with pytest.raises(fve.SmoeError):   # beyond the one-workgroup limits
        fve.moe_route_plan(dev(synth.tokens(synth.DS, 64)), dev(synth.router(synth.DS)),
                           synth.DS.k)


# ------------------------------------------------------------- S4 / S6 ----

_layers = {}


def _layer(shape, Ts, steps=(0,), int4=True, f16=True):
    key = (shape.name, Ts, steps, int4, f16)
    if key not in _layers:
        xs = [synth.tokens(shape, T, step=st) for T in Ts for st in steps]
        _layers[key] = Layer(shape, xs, int4=int4, f16=f16)
    return _layers[key]


# long reductions: three and four 128-K groups per slot in the one-token path
_LONG_I = dataclasses.replace(synth.TINY, name="tiny_i12288", E=4, k=2, I=12288)
_LONG_H = dataclasses.replace(synth.TINY, name="tiny_h16384", H=16384, E=4, k=2, I=256)
W4_CASES = [(synth.TINY, 4), (synth.TINY, 40), (synth.DS, 1), (synth.DS, 4), (synth.DS, 16),
            (synth.PHI, 1), (synth.QWEN, 1), (_LONG_I, 1), (_LONG_I, 3), (_LONG_H, 1),
            (_LONG_H, 2)]


@pytest.mark.parametrize("shape,T", W4_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_w4a16_grouped_ffn(shape, T):
    say(f"w4a16 {shape.name} T={T}")
    L = _layer(shape, (T,), f16=False)
    x = synth.tokens(shape, T, step=0)
    r = oracle.route_topk(x, L.router, shape.k)
    maps = oracle.gather_maps(r["ids"], shape.E)
    ref = oracle.grouped_ffn(x, maps, L.int4, "int4")
    err = _err()
    dx = dev(x)
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, shape.k)
    gm = fve.moe_gather(ids, shape.E, err)
    ws = fve.new_workspace(0, T, shape.k, shape.H, shape.I, shape.E)
    y = fve.w4a16_grouped_ffn(dx, gm, L.t4, T, shape.k, shape.H, shape.I, shape.E, ws,
                              err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    rows = T * shape.k
    st = assert_fp16_close(host(y)[:rows], ref, f"w4a16 {shape.name} T={T}")
    say(f"  l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")
    # deterministic: a second call gives the same bits; counters reset
    y2 = fve.w4a16_grouped_ffn(dx, gm, L.t4, T, shape.k, shape.H, shape.I, shape.E, ws,
                               err_word=err)
    assert torch.equal(y[:rows], y2[:rows])


# Other draft code widths (2 and 8 bits, GPTQ layout).
_WIDE_Q = dataclasses.replace(synth.TINY, name="tiny_e128_k5", E=128, k=5)   # > 64 experts
WQ_CASES = [(synth.TINY, 1, 2), (synth.TINY, 1, 8), (synth.TINY, 40, 2), (synth.TINY, 40, 8),
            (synth.DS, 1, 8), (synth.DS, 4, 2), (synth.DS, 16, 8), (synth.PHI, 1, 2),
            (synth.PHI, 1, 8), (synth.QWEN, 1, 8), (_LONG_I, 1, 8), (_LONG_H, 1, 2),
            (_LONG_H, 3, 8), (_WIDE_Q, 1, 8), (_WIDE_Q, 5, 2)]


@pytest.mark.parametrize("shape,T,bits", WQ_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_wq_grouped_ffn(shape, T, bits):
    """wq_grouped_ffn at 2 and 8 bits against the oracle (the long 8-bit
    reductions take the multi-row kernels at T = 1: more than four
    pseudo-groups per slot)."""
    say(f"wq{bits} {shape.name} T={T}")
    E, k = shape.E, shape.k
    x = synth.tokens(shape, T, step=1)
    router = synth.router(shape)
    r = oracle.route_topk(x, router, k)
    touched = sorted(set(int(e) for e in r["ids"].ravel()))
    q = [None] * E
    for e in touched:
        q[e] = synth.expert_int4(*synth.expert_f16(shape, 0, e), bits=bits)
    table, _keep = upload_int4(q)
    maps = oracle.gather_maps(r["ids"], E)
    ref = oracle.grouped_ffn(x, maps, q, f"int{bits}")
    err = _err()
    dx = dev(x)
    ids, _, _ = fve.moe_route_topk(dx, dev(router), k)
    gm = fve.moe_gather(ids, E, err)
    ws = fve.new_workspace(0, T, k, shape.H, shape.I, E)
    y = fve.wq_grouped_ffn(dx, gm, table, T, k, shape.H, shape.I, E, ws, bits, err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    rows = T * k
    st = assert_fp16_close(host(y)[:rows], ref, f"wq{bits} {shape.name} T={T}")
    say(f"  l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")
    y2 = fve.wq_grouped_ffn(dx, gm, table, T, k, shape.H, shape.I, E, ws, bits, err_word=err)
    assert torch.equal(y[:rows], y2[:rows])


def test_wq_bits4_is_w4a16():
    s = synth.DS
    L = _layer(s, (4,), f16=False)
    x = dev(synth.tokens(s, 4, step=0))
    ids, _, _ = fve.moe_route_topk(x, L.d_router, s.k)
    gm = fve.moe_gather(ids, s.E)
    ws = fve.new_workspace(0, 4, s.k, s.H, s.I, s.E)
    a = fve.w4a16_grouped_ffn(x, gm, L.t4, 4, s.k, s.H, s.I, s.E, ws)
    b = fve.wq_grouped_ffn(x, gm, L.t4, 4, s.k, s.H, s.I, s.E, ws, 4)
    assert torch.equal(a[:4 * s.k], b[:4 * s.k])
    with pytest.raises(fve.SmoeError):
        fve.wq_grouped_ffn(x, gm, L.t4, 4, s.k, s.H, s.I, s.E, ws, 3)


# One-token draft step with the routing folded into the gate/up launch.
_WIDE = dataclasses.replace(synth.TINY, name="tiny_e128_k5", E=128, k=5)   # > 64 experts
_ALL = dataclasses.replace(synth.TINY, name="tiny_k_eq_e", k=8)            # every expert
_RENORM = dataclasses.replace(synth.TINY, name="tiny_renorm_k3", k=3, renormalize=True)
DRAFT_FUSED_CASES = [(synth.TINY, 0), (synth.TINY, 7), (synth.DS, 0), (synth.DS, 3),
                     (synth.QWEN, 0), (synth.PHI, 0), (synth.PHI, 5), (_WIDE, 0), (_ALL, 0),
                     (_RENORM, 2), (_LONG_I, 0), (_LONG_H, 1), (_E256, 0), (_E256, 4)]


@pytest.mark.parametrize("shape,step", DRAFT_FUSED_CASES,
                         ids=lambda v: getattr(v, "name", str(v)))
def test_draft_route_ffn_matches_separate_calls(shape, step):
    """moe_draft_route_ffn equals moe_route_plan + w4a16_grouped_ffn bit for
    bit (ids, weights, gate, ELB row, maps, y_sorted), and the oracle."""
    say(f"draft route+ffn {shape.name} step={step}")
    E, k = shape.E, shape.k
    x = synth.tokens(shape, 1, step=step)
    L = _layer(shape, (1,), steps=(step,), f16=False)
    dx = dev(x)
    c0 = np.random.default_rng(step).integers(0, 50, size=(3, E)).astype(np.int32)
    counters, counters2 = dev(c0), dev(c0)
    err = _err()
    ws = fve.new_workspace(0, 1, k, shape.H, shape.I, E)
    ids, w, gate, m, y = fve.moe_draft_route_ffn(dx, L.d_router, k, L.t4, shape.I, ws,
                                                 shape.renormalize, L.d_gate,
                                                 counters=counters, layer=2, err_word=err)
    ids2, w2, gate2, m2 = fve.moe_route_plan(dx, L.d_router, k, shape.renormalize, L.d_gate,
                                             counters=counters2, layer=2)
    ws2 = fve.new_workspace(0, 1, k, shape.H, shape.I, E)
    y2 = fve.w4a16_grouped_ffn(dx, m2, L.t4, 1, k, shape.H, shape.I, E, ws2)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert torch.equal(ids, ids2)
    assert torch.equal(w, w2)
    if L.d_gate is not None:
        assert torch.equal(gate, gate2)
    assert torch.equal(counters, counters2)
    for key in ("offsets", "active", "n_active"):
        assert torch.equal(m[key], m2[key]), key
    for key in ("sorted_token", "sorted_pair", "pair_pos"):
        assert torch.equal(m[key][:k], m2[key][:k]), key
    assert torch.equal(y[:k], y2[:k])
    ref = oracle.route_topk(x, L.router, k, shape.renormalize)
    assert np.array_equal(host(ids), ref["ids"])
    assert np.allclose(host(w), ref["weights"], rtol=W_RTOL, atol=1e-7)
    assert np.array_equal(host(counters), oracle.elb_update(c0, ref["ids"], 2))
    maps = oracle.gather_maps(ref["ids"], E)
    assert np.array_equal(host(m["offsets"]), maps["offsets"])
    assert np.array_equal(host(m["sorted_pair"])[:k], maps["sorted_pair"])
    yref = oracle.grouped_ffn(x, maps, L.int4, "int4")
    st = assert_fp16_close(host(y)[:k], yref, f"draft route+ffn {shape.name}")
    say(f"  l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")


def test_draft_route_ffn_nan_logit_and_repeat():
    """A NaN logit ranks last in the fused routing too; a second call on the
    same inputs gives the same bits and adds the same ELB increments again."""
    s = _ALL
    x = synth.tokens(s, 1, step=4)
    L = _layer(s, (1,), steps=(4,), f16=False)
    wr = L.router.copy()
    wr[5, 0] = np.float16(np.inf)
    x[:, 0] = 0.0                                     # 0 * inf: expert 5's logit is NaN
    ws = fve.new_workspace(0, 1, s.k, s.H, s.I, s.E)
    counters = torch.zeros((1, s.E), dtype=torch.int32, device="cuda")
    ids, w, _, m, y = fve.moe_draft_route_ffn(dev(x), dev(wr), s.k, L.t4, s.I, ws,
                                              counters=counters)
    ref = oracle.route_topk(x, wr, s.k)
    assert np.array_equal(host(ids), ref["ids"])
    assert host(ids)[0, -1] == 5
    y1 = y.clone()
    fve.moe_draft_route_ffn(dev(x), dev(wr), s.k, L.t4, s.I, ws, counters=counters,
                            topk_ids=ids, topk_w=w, maps=m, y_sorted=y)
    assert torch.equal(y, y1)
    assert host(counters).tolist() == [[2] * s.E]
    # without counters: no ELB update, the same outputs
    ids2, w2, _, m2, y2 = fve.moe_draft_route_ffn(dev(x), dev(wr), s.k, L.t4, s.I, ws)
    # (the NaN logit makes every softmax weight NaN, as in the oracle)
    assert torch.isnan(w).all() and torch.isnan(w2).all()
    assert torch.equal(ids2, ids) and torch.equal(y2[:s.k], y1[:s.k])
    assert torch.equal(m2["offsets"], m["offsets"])


# The dense shared expert inside the one-token draft launches: fused into the
# gate/up and down launches at the DeepSeek, Qwen and (H = 4096) Phi-like
# shapes, launches of its own for the tiny one (no fused instantiation).
_TINY_SHD = dataclasses.replace(synth.TINY, name="tiny_shared_draft", shared_I=384)
_PHI_SHD = dataclasses.replace(synth.PHI, name="phi_shared_draft", shared_I=4096,
                               shared_gate=True)
DRAFT_SHARED_CASES = [(synth.DS, 0), (synth.DS, 2), (synth.QWEN, 0), (synth.QWEN, 5),
                      (_TINY_SHD, 1), (_PHI_SHD, 0)]


@pytest.mark.parametrize("shape,step", DRAFT_SHARED_CASES,
                         ids=lambda v: getattr(v, "name", str(v)))
def test_draft_route_ffn_shared_expert(shape, step):
    """With a shared expert, moe_draft_route_ffn leaves every routed output
    bit-identical to the call without one, and its shared output equals
    verify_grouped_gemm on the same row bit for bit (and the oracle)."""
    say(f"draft route+ffn with shared expert {shape.name} step={step}")
    E, k, H, I, Is = shape.E, shape.k, shape.H, shape.I, shape.shared_I
    x = synth.tokens(shape, 1, step=step)
    L = _layer(shape, (1,), steps=(step,), f16=False)
    assert L.shared is not None
    dx = dev(x)
    err = _err()
    counters = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    counters2 = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    ws = fve.new_workspace(0, 1, k, H, I, E)
    shared = (dev(L.shared["w13"]), dev(L.shared["w2"]))
    ids, w, gate, m, y, so = fve.moe_draft_route_ffn(dx, L.d_router, k, L.t4, I, ws,
                                                     shape.renormalize, L.d_gate,
                                                     counters=counters, err_word=err,
                                                     shared=shared)
    ws2 = fve.new_workspace(0, 1, k, H, I, E)
    ids2, w2, gate2, m2, y2 = fve.moe_draft_route_ffn(dx, L.d_router, k, L.t4, I, ws2,
                                                      shape.renormalize, L.d_gate,
                                                      counters=counters2)
    iota = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    wsv = fve.new_workspace(1, 1, 1, H, Is, 1)
    yv = fve.verify_grouped_gemm(dx, iota, offs, L.tsh, 1, 1, H, Is, 1, wsv)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(counters, counters2)
    if L.d_gate is not None:
        assert torch.equal(gate, gate2)
    for key in ("offsets", "active", "n_active"):
        assert torch.equal(m[key], m2[key]), key
    for key in ("sorted_token", "sorted_pair", "pair_pos"):
        assert torch.equal(m[key][:k], m2[key][:k]), key
    assert torch.equal(y[:k], y2[:k])
    assert torch.equal(so, yv[:1]), "shared output differs from verify_grouped_gemm"
    ref = oracle.expert_ffn_f16(x, L.shared["w13"], L.shared["w2"])
    st = assert_fp16_close(host(so), ref, f"draft shared {shape.name}")
    say(f"  shared l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")


# AWQ-style experts: per-input-channel divisors on both projections' inputs.
AWQ_CASES = [(synth.TINY, 1), (synth.TINY, 4), (synth.TINY, 40), (synth.DS, 1), (synth.DS, 4),
             (synth.PHI, 1), (synth.QWEN, 1)]


def _awq_layer(shape, T, step):
    L = _layer(shape, (T,), steps=(step,), f16=False)
    ex = [None] * shape.E
    for e in L.touched:
        ex[e] = synth.expert_awq(shape, 0, e, *L.f16[e])
    gpu = [None if a is None else {key: tuple(dev(t) for t in a[key]) for key in ("w13", "w2")}
           for a in ex]
    sc = [None if a is None else (dev(a["a13"]), dev(a["a2"])) for a in ex]
    return L, ex, gpu, sc


@pytest.mark.parametrize("shape,T", AWQ_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_awq_grouped_ffn(shape, T):
    say(f"awq {shape.name} T={T}")
    E, k, H, I = shape.E, shape.k, shape.H, shape.I
    step = 5
    L, ex, gpu, sc = _awq_layer(shape, T, step)
    table = fve.w4_expert_table(gpu)
    stab = fve.awq_scale_table(sc)
    x = synth.tokens(shape, T, step=step)
    r = oracle.route_topk(x, L.router, k)
    ref = oracle.grouped_ffn(x, oracle.gather_maps(r["ids"], E), ex, "awq")
    dx = dev(x)
    err = _err()
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, k)
    gm = fve.moe_gather(ids, E, err)
    ws = fve.new_workspace(0, T, k, H, I, E)
    y = fve.awq_grouped_ffn(dx, gm, table, stab, T, k, H, I, E, ws, err_word=err)
    y2 = fve.awq_grouped_ffn(dx, gm, table, stab, T, k, H, I, E, ws, err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    rows = T * k
    st = assert_fp16_close(host(y)[:rows], ref, f"awq {shape.name} T={T}")
    assert torch.equal(y[:rows], y2[:rows])
    say(f"  l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")


def test_awq_unit_factors_are_w4a16_and_null_flagged():
    """Unit divisors leave the one-token step bit-identical to
    w4a16_grouped_ffn on the same codes; a touched expert without divisors is
    skipped and flagged."""
    s = synth.DS
    E, k, H, I = s.E, s.k, s.H, s.I
    L = _layer(s, (1,), steps=(0,), f16=False)
    ones = (torch.ones(H, dtype=torch.float16, device="cuda"),
            torch.ones(I, dtype=torch.float16, device="cuda"))
    stab = fve.awq_scale_table([ones if e in L.touched else None for e in range(E)])
    x = dev(synth.tokens(s, 1, step=0))
    err = _err()
    ids, _, _ = fve.moe_route_topk(x, L.d_router, k)
    gm = fve.moe_gather(ids, E, err)
    ws = fve.new_workspace(0, 1, k, H, I, E)
    a = fve.awq_grouped_ffn(x, gm, L.t4, stab, 1, k, H, I, E, ws, err_word=err)
    b = fve.w4a16_grouped_ffn(x, gm, L.t4, 1, k, H, I, E, ws, err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert torch.equal(a[:k], b[:k])
    # the first touched expert loses its divisors
    first = int(host(ids).ravel().min())
    stab2 = fve.awq_scale_table([ones if (e in L.touched and e != first) else None
                                 for e in range(E)])
    fve.awq_grouped_ffn(x, gm, L.t4, stab2, 1, k, H, I, E, ws, err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) & fve.SMOE_DERR_NULL_EXPERT


# The combine of one layer fused with the next layer's router logits.
COMBINE_LOGITS_CASES = [(synth.TINY, 0), (synth.DS, 1), (synth.QWEN, 2), (synth.PHI, 3),
                        (_E256, 4)]


@pytest.mark.parametrize("shape,step", COMBINE_LOGITS_CASES,
                         ids=lambda v: getattr(v, "name", str(v)))
def test_combine_route_logits_matches_separate_calls(shape, step):
    """moe_combine_route_logits: out and norm_out bit-identical to
    moe_combine's; the logits bit-identical to the oracle's pinned-order fp32
    logits of norm_out and to those moe_draft_route_ffn computes itself; and
    the next layer's draft step from the passed logits bit-identical to the
    step that computes them."""
    say(f"combine + next logits {shape.name} step={step}")
    E, k, H, I = shape.E, shape.k, shape.H, shape.I
    g = synth.torch_layer(shape, 0, "cuda", int4=True)
    g2 = synth.torch_layer(shape, 1, "cuda", int4=True)
    t4, t4b = fve.w4_expert_table(g["int4"]), fve.w4_expert_table(g2["int4"])
    sh = None if g["shared"] is None else (g["shared"]["w13"], g["shared"]["w2"])
    gate = None if g["shared"] is None else g["shared"]["gate"]
    sh2 = None if g2["shared"] is None else (g2["shared"]["w13"], g2["shared"]["w2"])
    gate2 = None if g2["shared"] is None else g2["shared"]["gate"]
    x = dev(synth.tokens(shape, 1, step=step))
    err = _err()
    ws = fve.new_workspace(0, 1, k, H, I, E)
    res = fve.moe_draft_route_ffn(x, g["router"], k, t4, I, ws, shape.renormalize, gate,
                                  err_word=err, shared=sh)
    ids, w, gt, m, y = res[:5]
    so = res[5] if sh is not None else None
    out_r, xn_r = fve.moe_combine(y, m["pair_pos"], w, so, gt, x, norm_out=True)
    out_f, xn_f, lg = fve.moe_combine_route_logits(y, m["pair_pos"], w, g2["router"], so, gt, x,
                                                   gate2)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_r) and torch.equal(xn_f, xn_r)
    ref_lg = oracle.logits_pinned_f32(host(xn_r), host(g2["router"]))[0]
    nv = E + (1 if gate2 is not None else 0)
    assert lg.shape[0] == nv
    assert np.array_equal(host(lg)[:E].view(np.uint32), ref_lg.view(np.uint32))
    if gate2 is not None:
        ref_g = oracle.logits_pinned_f32(host(xn_r), host(gate2))
        assert host(lg)[E].view(np.uint32) == np.float32(ref_g[0]).view(np.uint32)
    # the next layer's draft step with and without the passed logits
    c1 = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    c2 = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    wsa = fve.new_workspace(0, 1, k, H, I, E)
    wsb = fve.new_workspace(0, 1, k, H, I, E)
    ra = fve.moe_draft_route_ffn(xn_r, g2["router"], k, t4b, I, wsa, shape.renormalize, gate2,
                                 counters=c1, err_word=err, shared=sh2)
    rb = fve.moe_draft_route_ffn(xn_f, g2["router"], k, t4b, I, wsb, shape.renormalize, gate2,
                                 counters=c2, err_word=err, shared=sh2, logits=lg)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    # the logits the step computed itself sit in its workspace after h and the slot table
    off = ((k * I * 2 + 255) // 256) * 256 + ((min(E, k) * 32 + 255) // 256) * 256
    own = wsa[off:off + 4 * nv].view(torch.float32)
    assert torch.equal(own, lg)
    assert torch.equal(ra[0], rb[0]) and torch.equal(ra[1], rb[1]) and torch.equal(c1, c2)
    if gate2 is not None:
        assert torch.equal(ra[2], rb[2])
    for key in ("offsets", "active", "n_active"):
        assert torch.equal(ra[3][key], rb[3][key]), key
    assert torch.equal(ra[4][:k], rb[4][:k])
    if sh2 is not None:
        assert torch.equal(ra[5], rb[5])


VERIFY_CASES = [(synth.TINY, 17), (synth.TINY, 40), (synth.QWEN, 9), (synth.PHI, 17),
                (synth.DS, 16),
                # T <= 4: the one-wave-per-column kernel (1, 2 and 4 rows per block)
                (synth.TINY, 1), (synth.TINY, 3), (synth.QWEN, 1), (synth.DS, 2),
                (synth.QWEN, 4), (synth.PHI, 1),
                # the largest reductions: hidden 16384 (past the matrix-vector
                # kernel's 8192, so MFMA even at T = 1) and intermediate 12288
                (_LONG_H, 1), (_LONG_H, 9), (_LONG_I, 3), (_LONG_I, 17)]


@pytest.mark.parametrize("shape,T", VERIFY_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_verify_grouped_gemm(shape, T):
    say(f"verify {shape.name} T={T}")
    L = _layer(shape, (T,), int4=False)
    x = synth.tokens(shape, T, step=0)
    r = oracle.route_topk(x, L.router, shape.k)
    maps = oracle.gather_maps(r["ids"], shape.E)
    ref = oracle.grouped_ffn(x, maps, L.f16, "f16")
    err = _err()
    dx = dev(x)
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, shape.k)
    gm = fve.moe_gather(ids, shape.E, err)
    ws = fve.new_workspace(1, T, shape.k, shape.H, shape.I, shape.E)
    rows = T * shape.k
    y = fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], L.t16, T, rows, shape.H,
                                shape.I, shape.E, ws, active=gm["active"],
                                n_active=gm["n_active"], err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    st = assert_fp16_close(host(y)[:rows], ref, f"verify {shape.name} T={T}")
    say(f"  l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")
    # the regrouped result equals the per-token GEMV ordering
    if shape.name in ("qwen15_moe", "tiny"):
        pt = oracle.per_token_ffn(x, r["ids"], L.f16, "f16")
        yy = host(y).astype(np.float64)
        per = np.stack([yy[maps["pair_pos"][t * shape.k:(t + 1) * shape.k]] for t in range(T)])
        assert_fp16_close(per, pt, "verify vs per-token ordering")
    # without the active list (scan all E) the result is bit-identical
    y2 = fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], L.t16, T, rows, shape.H,
                                 shape.I, shape.E, ws, err_word=err)
    assert torch.equal(y[:rows], y2[:rows])


# dense regime (many rows per expert): the tiled grouped GEMM
# hidden 384: a last, partial 256-column block in the down projection
_H384 = dataclasses.replace(synth.TINY, name="tiny_h384", H=384, E=4, k=2, I=256)
DENSE_CASES = [(synth.TINY, 512, None), (synth.TINY, 300, None), (synth.DS, 700, 40),
               (synth.PHI, 2048, 24), (_H384, 512, None)]


def _sample_tokens(T, n):
    """n tokens spread over [0, T), first and last included (None = all)."""
    if n is None or n >= T:
        return np.arange(T)
    return np.unique(np.linspace(0, T - 1, n).round().astype(np.int64))


@pytest.mark.parametrize("shape,T,sample", DENSE_CASES,
                         ids=lambda v: getattr(v, "name", str(v)))
def test_verify_dense_regime(shape, T, sample):
    """Mean rows per expert >= 64: the tiled GEMM.  Small cases against the
    whole grouped oracle; the large ones (the Phi T = 2048 point timed by
    bench.py among them) on sampled tokens computed one by one."""
    say(f"verify dense {shape.name} T={T}")
    L = _layer(shape, (T,), int4=False)
    x = synth.tokens(shape, T, step=0)
    r = oracle.route_topk(x, L.router, shape.k)
    maps = oracle.gather_maps(r["ids"], shape.E)
    err = _err()
    dx = dev(x)
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, shape.k)
    gm = fve.moe_gather(ids, shape.E, err)
    assert np.array_equal(host(ids), r["ids"])
    ws = fve.new_workspace(1, T, shape.k, shape.H, shape.I, shape.E)
    rows = T * shape.k
    y = fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], L.t16, T, rows, shape.H,
                                shape.I, shape.E, ws, active=gm["active"],
                                n_active=gm["n_active"], err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    yy = host(y)
    toks = _sample_tokens(T, sample)
    if sample is None:
        ref = oracle.grouped_ffn(x, maps, L.f16, "f16")
        st = assert_fp16_close(yy[:rows], ref, f"dense {shape.name} T={T}")
    else:
        pt = oracle.per_token_ffn(x[toks], r["ids"][toks], L.f16, "f16")
        got = np.stack([yy[maps["pair_pos"][t * shape.k:(t + 1) * shape.k]] for t in toks])
        st = assert_fp16_close(got, pt, f"dense {shape.name} T={T} sampled")
    say(f"  l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")
    # deterministic, and the active list is optional
    y2 = fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], L.t16, T, rows, shape.H,
                                 shape.I, shape.E, ws, err_word=err)
    assert torch.equal(y[:rows], y2[:rows])


def test_verify_dense_mask_and_skew():
    """Dense regime: hits then misses == all at once (bit-identical), and a
    skewed routing where one expert holds most rows (many row tiles)."""
    s, T = synth.TINY, 600
    rng = np.random.default_rng(11)
    ids = np.empty((T, s.k), np.int32)
    for t in range(T):
        a = 0 if rng.random() < 0.8 else int(rng.integers(1, s.E))
        b = int(rng.integers(0, s.E - 1))
        ids[t] = (a, b if b < a else b + 1)
    data = synth.make_layer(s, 0, int4=False, f16=True)
    t16, keep = upload_f16(data["f16"])
    x = synth.tokens(s, T, step=4)
    maps = oracle.gather_maps(ids, s.E)
    assert maps["offsets"][1] - maps["offsets"][0] > 400          # expert 0: 4+ row tiles
    ref = oracle.grouped_ffn(x, maps, data["f16"], "f16")
    dx = dev(x)
    gm = fve.moe_gather(dev(ids), s.E)
    rows = T * s.k
    ws = fve.new_workspace(1, T, s.k, s.H, s.I, s.E)
    full = fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], t16, T, rows, s.H, s.I,
                                   s.E, ws, active=gm["active"], n_active=gm["n_active"])
    torch.cuda.synchronize()
    assert_fp16_close(host(full)[:rows], ref, "dense skewed")
    hit = torch.zeros(s.E, dtype=torch.uint8, device="cuda")
    hit[0] = 1
    hit[3] = 1
    y = torch.full_like(full, float("nan"))
    for m in (hit, 1 - hit):
        fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], t16, T, rows, s.H, s.I,
                                s.E, ws, active=gm["active"], n_active=gm["n_active"],
                                expert_mask=m, y_sorted=y)
    assert torch.equal(y[:rows], full[:rows])
    del keep


def test_verify_dense_forms_bit_identical():
    """The dense regime's two forms of the tile -- the global->LDS ring (at
    least a full 128-row tile per expert on average) and the register-staged
    form -- give the same bits: the same routed rows declared over 8 experts
    (1024 rows: the ring) and over 16 whose last 8 are empty (the register
    form), both against the oracle too."""
    s, T = synth.TINY, 512
    data = synth.make_layer(s, 0, int4=False, f16=True)
    t16, keep = upload_f16(data["f16"])
    t16b, keep_b = upload_f16(list(data["f16"]) + [data["f16"][0]] * s.E)  # 8-15 never touched
    x = synth.tokens(s, T, step=5)
    rng = np.random.default_rng(12)
    ids = np.stack([rng.permutation(s.E)[:s.k] for _ in range(T)]).astype(np.int32)
    dx = dev(x)
    gm = fve.moe_gather(dev(ids), s.E)
    rows = T * s.k
    assert rows >= 128 * s.E and rows < 128 * 2 * s.E
    ws = fve.new_workspace(1, T, s.k, s.H, s.I, s.E)
    ring = fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], t16, T, rows, s.H,
                                   s.I, s.E, ws)
    off2 = torch.cat([gm["offsets"], gm["offsets"][-1:].repeat(s.E)])
    ws2 = fve.new_workspace(1, T, s.k, s.H, s.I, 2 * s.E)
    reg = fve.verify_grouped_gemm(dx, gm["sorted_token"], off2, t16b, T, rows, s.H, s.I,
                                  2 * s.E, ws2)
    torch.cuda.synchronize()
    assert torch.equal(ring[:rows], reg[:rows])
    ref = oracle.grouped_ffn(x, oracle.gather_maps(ids, s.E), data["f16"], "f16")
    assert_fp16_close(host(ring)[:rows], ref, "dense forms")
    del keep, keep_b


def test_shared_expert_dense():
    """A shared expert over 128 rows (one group of T rows): dense regime."""
    s, T = synth.QWEN, 128
    sh = synth.shared_expert(s)
    tsh, keep = upload_f16([(sh["w13"], sh["w2"])])
    x = synth.tokens(s, T, step=6)
    ws = fve.new_workspace(1, T, 1, s.H, s.shared_I, 1)
    iota = torch.arange(T, dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    y = fve.verify_grouped_gemm(dev(x), iota, offs, tsh, T, T, s.H, s.shared_I, 1, ws)
    torch.cuda.synchronize()
    toks = _sample_tokens(T, 32)
    ref = oracle.expert_ffn_f16(x[toks], sh["w13"], sh["w2"])
    assert_fp16_close(host(y)[toks], ref, "shared dense")
    del keep


def test_verify_expert_mask_hits_then_misses():
    s, T = synth.QWEN, 9
    L = _layer(s, (T,), int4=False)
    x = dev(synth.tokens(s, T, step=0))
    ids, _, _ = fve.moe_route_topk(x, L.d_router, s.k)
    gm = fve.moe_gather(ids, s.E)
    ws = fve.new_workspace(1, T, s.k, s.H, s.I, s.E)
    rows = T * s.k
    full = fve.verify_grouped_gemm(x, gm["sorted_token"], gm["offsets"], L.t16, T, rows, s.H,
                                   s.I, s.E, ws, active=gm["active"], n_active=gm["n_active"])
    hit = torch.zeros(s.E, dtype=torch.uint8, device="cuda")
    hit[torch.tensor(L.touched[::2])] = 1
    miss = 1 - hit
    y = torch.full_like(full, float("nan"))
    fve.verify_grouped_gemm(x, gm["sorted_token"], gm["offsets"], L.t16, T, rows, s.H, s.I, s.E,
                            ws, active=gm["active"], n_active=gm["n_active"], expert_mask=hit,
                            y_sorted=y)
    fve.verify_grouped_gemm(x, gm["sorted_token"], gm["offsets"], L.t16, T, rows, s.H, s.I, s.E,
                            ws, active=gm["active"], n_active=gm["n_active"], expert_mask=miss,
                            y_sorted=y)
    assert torch.equal(y[:rows], full[:rows])


def test_null_expert_flagged():
    s, T = synth.TINY, 4
    L = _layer(s, (T,))
    x = dev(synth.tokens(s, T, step=0))
    ids, _, _ = fve.moe_route_topk(x, L.d_router, s.k)
    gm = fve.moe_gather(ids, s.E)
    e0 = L.touched[0]
    t4 = L.t4.clone()
    t4[e0] = 0
    t16 = L.t16.clone()
    t16[e0] = 0
    for kind in ("int4", "f16"):
        err = _err()
        if kind == "int4":
            ws = fve.new_workspace(0, T, s.k, s.H, s.I, s.E)
            fve.w4a16_grouped_ffn(x, gm, t4, T, s.k, s.H, s.I, s.E, ws, err_word=err)
        else:
            ws = fve.new_workspace(1, T, s.k, s.H, s.I, s.E)
            fve.verify_grouped_gemm(x, gm["sorted_token"], gm["offsets"], t16, T, T * s.k, s.H,
                                    s.I, s.E, ws, active=gm["active"], n_active=gm["n_active"],
                                    err_word=err)
        assert int(host(err)[0]) & fve.SMOE_DERR_NULL_EXPERT


# ---------------------------------------------------------------- S5 ----

_TINY_SH = dataclasses.replace(synth.TINY, name="tiny_shared", shared_I=384)


@pytest.mark.parametrize("shape,T", [(synth.DS, 1), (synth.DS, 16), (synth.QWEN, 9),
                                     (synth.QWEN, 17), (synth.QWEN, 1), (synth.QWEN, 4),
                                     (synth.DS, 3), (_TINY_SH, 1), (_TINY_SH, 2)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_shared_expert(shape, T):
    sh = synth.shared_expert(shape)
    x = synth.tokens(shape, T, step=1)
    ref = oracle.expert_ffn_f16(x, sh["w13"], sh["w2"])
    from gpu_util import upload_f16
    tab, keep = upload_f16([(sh["w13"], sh["w2"])])
    dx = dev(x)
    iota = torch.arange(T, dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    ws = fve.new_workspace(1, T, 1, shape.H, shape.shared_I, 1)
    y = fve.verify_grouped_gemm(dx, iota, offs, tab, T, T, shape.H, shape.shared_I, 1, ws)
    assert_fp16_close(host(y)[:T], ref, f"shared {shape.name} T={T}")


# verify_grouped_gemm_shared: the shared expert's items inside the routed
# ring launches (Qwen T = 9, DeepSeek T = 16, a Phi-like H = 4096 layer with
# a shared expert: 2- and 4-wave rings), and the fallbacks (T = 3: the
# matrix-vector kernel; Qwen T = 17: a shared group longer than the routed
# launches' row block)
_PHI_SHV = dataclasses.replace(synth.PHI, name="phi_shared_verify", shared_I=4096,
                               shared_gate=True)
VERIFY_SHARED_CASES = [(synth.QWEN, 9), (synth.DS, 16), (_PHI_SHV, 9), (synth.QWEN, 3),
                       (synth.QWEN, 17)]


@pytest.mark.parametrize("shape,T", VERIFY_SHARED_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_verify_grouped_gemm_shared(shape, T):
    """The routed output bit-identical to verify_grouped_gemm's, the shared
    output within the bars of the oracle's FP16 shared expert; twice in a row
    on the same buffers (the second call may not depend on the first's)."""
    say(f"verify + shared {shape.name} T={T}")
    E, k, H, I, Is = shape.E, shape.k, shape.H, shape.I, shape.shared_I
    L = _layer(shape, (T,), steps=(2,), int4=False)
    x = synth.tokens(shape, T, step=2)
    dx = dev(x)
    err = _err()
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, k)
    gm = fve.moe_gather(ids, E, err)
    ws = fve.new_workspace(1, T, k, H, I, E)
    y_ref = fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], L.t16, T, T * k, H, I,
                                    E, ws, active=gm["active"], n_active=gm["n_active"])
    y_ref = y_ref.clone()
    shared = (dev(L.shared["w13"]), dev(L.shared["w2"]))
    ws2 = fve.new_workspace(1, T, k, H, I, E)
    ref_sh = oracle.expert_ffn_f16(x, L.shared["w13"], L.shared["w2"])
    for rep in range(2):
        y, so = fve.verify_grouped_gemm_shared(dx, gm["sorted_token"], gm["offsets"], L.t16, T,
                                               T * k, H, I, E, ws2, shared, active=gm["active"],
                                               n_active=gm["n_active"], err_word=err)
        torch.cuda.synchronize()
        assert int(host(err)[0]) == 0
        assert torch.equal(y[:T * k], y_ref[:T * k]), "routed rows differ from verify_grouped_gemm"
        st = assert_fp16_close(host(so), ref_sh, f"verify shared {shape.name} T={T}")
        if rep == 0:
            first = so.clone()
        else:
            assert torch.equal(so, first), "second call differs"
    say(f"  shared l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")


# DeepSeek: the shared columns inside the multi-row launches (T 2-4: the
# matrix-vector routine; T 5-16: MFMA items), then the one-expert ring
# kernels after them (T 17); Qwen (shared intermediate 5632): MFMA items
# (T 16), launches of their own after the multi-row (T 4) or one-token (T 1)
# launches; hidden and shared intermediate 4096 (8 chunks per lane both ways).
W4_SHARED_CASES = [(synth.DS, 2), (synth.DS, 4), (synth.DS, 5), (synth.DS, 9), (synth.DS, 16),
                   (synth.DS, 17), (synth.QWEN, 4), (synth.QWEN, 16), (synth.QWEN, 1),
                   (_PHI_SHV, 3), (_PHI_SHV, 9)]
# below 1024 the verify call takes other kernels for the lone shared expert:
# the shared output is held to the oracle only
_TINY_SH = dataclasses.replace(synth.TINY, name="tiny_shared", shared_I=384)


@pytest.mark.parametrize("shape,T", W4_SHARED_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_w4a16_grouped_ffn_shared(shape, T):
    """The routed output bit-identical to w4a16_grouped_ffn's; the shared
    expert's output bit-identical to verify_grouped_gemm's with the shared
    expert as its only expert over the T rows in order, and within the bars of
    the oracle's FP16 shared expert; twice in a row on the same buffers."""
    say(f"w4a16 + shared {shape.name} T={T}")
    E, k, H, I, Is = shape.E, shape.k, shape.H, shape.I, shape.shared_I
    L = _layer(shape, (T,), steps=(2,), f16=False)
    x = synth.tokens(shape, T, step=2)
    dx = dev(x)
    err = _err()
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, k)
    gm = fve.moe_gather(ids, E, err)
    ws = fve.new_workspace(0, T, k, H, I, E)
    y_ref = fve.w4a16_grouped_ffn(dx, gm, L.t4, T, k, H, I, E, ws).clone()
    shared = (dev(L.shared["w13"]), dev(L.shared["w2"]))
    iota = torch.arange(T, dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    wsv = fve.new_workspace(1, T, 1, H, Is, 1)
    so_ref = fve.verify_grouped_gemm(dx, iota, offs, L.tsh, T, T, H, Is, 1, wsv).clone()
    ref_sh = oracle.expert_ffn_f16(x, L.shared["w13"], L.shared["w2"])
    ws2 = fve.new_workspace(0, T, k, H, I, E)
    for rep in range(2):
        y, so = fve.w4a16_grouped_ffn_shared(dx, gm, L.t4, T, k, H, I, E, ws2, shared,
                                             err_word=err)
        torch.cuda.synchronize()
        assert int(host(err)[0]) == 0
        assert torch.equal(y[:T * k], y_ref[:T * k]), "routed rows differ from w4a16_grouped_ffn"
        assert torch.equal(so, so_ref[:T]), "shared expert differs from verify_grouped_gemm"
        st = assert_fp16_close(host(so), ref_sh, f"w4a16 shared {shape.name} T={T}")
        if rep == 0:
            first = so.clone()
        else:
            assert torch.equal(so, first), "second call differs"
    say(f"  shared l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")


@pytest.mark.parametrize("T", [3, 9, 20])
def test_w4a16_grouped_ffn_shared_small(T):
    """Hidden 256 and shared intermediate 384: the standalone matrix-vector
    launches (T 3) and the one-group ring launches (T 9, 20) after the routed
    ones; routed rows bit-identical to w4a16_grouped_ffn's, the shared expert
    within the bars of the oracle's."""
    shape = _TINY_SH
    say(f"w4a16 + shared {shape.name} T={T}")
    E, k, H, I, Is = shape.E, shape.k, shape.H, shape.I, shape.shared_I
    L = _layer(shape, (T,), steps=(2,), f16=False)
    x = synth.tokens(shape, T, step=2)
    dx = dev(x)
    err = _err()
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, k)
    gm = fve.moe_gather(ids, E, err)
    ws = fve.new_workspace(0, T, k, H, I, E)
    y_ref = fve.w4a16_grouped_ffn(dx, gm, L.t4, T, k, H, I, E, ws).clone()
    shared = (dev(L.shared["w13"]), dev(L.shared["w2"]))
    ref_sh = oracle.expert_ffn_f16(x, L.shared["w13"], L.shared["w2"])
    y, so = fve.w4a16_grouped_ffn_shared(dx, gm, L.t4, T, k, H, I, E, ws, shared, err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert torch.equal(y[:T * k], y_ref[:T * k])
    if T <= 4:  # both calls take the matrix-vector routine at any size
        iota = torch.arange(T, dtype=torch.int32, device="cuda")
        offs = torch.tensor([0, T], dtype=torch.int32, device="cuda")
        wsv = fve.new_workspace(1, T, 1, H, Is, 1)
        so_ref = fve.verify_grouped_gemm(dx, iota, offs, L.tsh, T, T, H, Is, 1, wsv)
        assert torch.equal(so, so_ref[:T])
    st = assert_fp16_close(host(so), ref_sh, f"w4a16 shared {shape.name} T={T}")
    say(f"  shared l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")


@pytest.mark.parametrize("T,rows", [(1, 3), (2, 5), (3, 9), (4, 4)])
def test_verify_few_tokens_long_groups(T, rows):
    """T <= 4 with an expert group longer than the kernel's row block (a
    token listed several times): every row is still FFN(x[token])."""
    shape = _TINY_SH
    sh = synth.shared_expert(shape)
    x = synth.tokens(shape, T, step=3)
    st = (np.arange(rows) * 7 + 1) % T
    ref = oracle.expert_ffn_f16(x[st], sh["w13"], sh["w2"])
    tab, keep = upload_f16([(sh["w13"], sh["w2"])])
    offs = torch.tensor([0, rows], dtype=torch.int32, device="cuda")
    ws = fve.new_workspace(1, T, rows, shape.H, shape.shared_I, 1)
    y = fve.verify_grouped_gemm(dev(x), dev(st.astype(np.int32)), offs, tab, T, rows, shape.H,
                                shape.shared_I, 1, ws)
    assert_fp16_close(host(y)[:rows], ref, f"few tokens T={T} rows={rows}")
    del keep


# ---------------------------------------------------------------- S7 ----

def test_combine():
    rng = np.random.default_rng(0)
    T, k, H = 9, 4, 2048
    y = rng.standard_normal((T * k, H)).astype(np.float16)
    pp = rng.permutation(T * k).astype(np.int32)
    pp[5] = -1
    w = rng.random((T, k)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float16)
    c = rng.random(T).astype(np.float32)
    res = rng.standard_normal((T, H)).astype(np.float16)
    ref = oracle.combine(y, pp, w.astype(np.float64), sh, c, res)
    out = fve.moe_combine(dev(y), dev(pp), dev(w), dev(sh), dev(c), dev(res))
    assert_fp16_close(host(out), ref, "combine", l2=1e-3, maxabs=4e-3)
    ref1 = oracle.combine(y, pp, w.astype(np.float64))
    out1 = fve.moe_combine(dev(y), dev(pp), dev(w))
    assert_fp16_close(host(out1), ref1, "combine plain", l2=1e-3, maxabs=4e-3)
    # fused RMS normalisation of the rounded output
    o, nrm = fve.moe_combine(dev(y), dev(pp), dev(w), dev(sh), dev(c), dev(res), norm_out=True)
    assert_fp16_close(host(nrm), oracle.rms_norm(host(o)), "combine norm", l2=1e-3, maxabs=4e-3)
    assert np.array_equal(host(o), host(out))
    # k = 1, weight 1: a permutation copy, exact
    pp1 = rng.permutation(T).astype(np.int32)
    out2 = fve.moe_combine(dev(y[:T]), dev(pp1), dev(np.ones((T, 1), np.float32)))
    assert np.array_equal(host(out2), y[:T][pp1])


@pytest.mark.parametrize("T,k", [(1, 2), (1, 6), (1, 8), (2, 4)])
def test_combine_few_rows(T, k):
    """Steps of at most 8 rows (one batch of slots): the oracle's sums, with a
    dropped pair and with the norm epilogue, and the same bits as the same
    tokens inside a step of more rows."""
    rng = np.random.default_rng(10 * T + k)
    H = 2048
    n = T * k
    y = rng.standard_normal((n, H)).astype(np.float16)
    pp = rng.permutation(n).astype(np.int32)
    pp[n - 1] = -1
    w = rng.random((T, k)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float16)
    c = rng.random(T).astype(np.float32)
    out, nrm = fve.moe_combine(dev(y), dev(pp), dev(w), dev(sh), dev(c), norm_out=True)
    ref = oracle.combine(y, pp, w.astype(np.float64), sh, c)
    assert_fp16_close(host(out), ref, "combine few rows", l2=1e-3, maxabs=4e-3)
    assert_fp16_close(host(nrm), oracle.rms_norm(host(out)), "combine few rows norm", l2=1e-3,
                      maxabs=4e-3)
    # the same tokens first in a step of more than 8 rows: the extra tokens'
    # rows follow, so the first T tokens' positions are unchanged
    X = 8 // k + 1
    y3 = np.concatenate([y, rng.standard_normal((X * k, H)).astype(np.float16)])
    pp3 = np.concatenate([pp, n + rng.permutation(X * k).astype(np.int32)])
    w3 = np.concatenate([w, rng.random((X, k)).astype(np.float32)])
    sh3 = np.concatenate([sh, rng.standard_normal((X, H)).astype(np.float16)])
    c3 = np.concatenate([c, rng.random(X).astype(np.float32)])
    assert (T + X) * k > 8
    out3 = fve.moe_combine(dev(y3), dev(pp3), dev(w3), dev(sh3), dev(c3))
    assert np.array_equal(host(out3)[:T], host(out))


# ----------------------------------------------------------- whole layer ----

LAYER_CASES = [(synth.TINY, 4, "int4"), (synth.DS, 1, "int4"), (synth.DS, 16, "int4"),
               (synth.QWEN, 9, "f16"), (synth.PHI, 1, "int4"), (synth.PHI, 17, "f16")]


@pytest.mark.parametrize("shape,T,kind", LAYER_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_layer_end_to_end(shape, T, kind):
    say(f"layer {shape.name} T={T} {kind}")
    L = _layer(shape, (T,), int4=(kind == "int4"), f16=(kind == "f16"))
    x = synth.tokens(shape, T, step=0)
    experts = L.int4 if kind == "int4" else L.f16
    shared = None if L.shared is None else dict(w13=L.shared["w13"], w2=L.shared["w2"],
                                                 gate=L.shared.get("gate"))
    ref = oracle.moe_layer(x, L.router, shape.k, experts, kind, shared)
    err = _err()
    got = run_layer(L, dev(x), kind, err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert np.array_equal(host(got["ids"]), ref["route"]["ids"])
    st = assert_fp16_close(host(got["out"]), ref["out"], f"layer {shape.name} T={T} {kind}")
    say(f"  l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")


@pytest.mark.parametrize("shape,T", [(synth.PHI, 20), (synth.PHI, 40), (synth.TINY, 100),
                                     (synth.QWEN, 33)], ids=lambda v: getattr(v, "name", str(v)))
def test_verify_one_expert_many_rows(shape, T):
    # one expert holding all T rows: 16/32-row blocks and several passes over
    # the weights, in both the short-reduction and the long-reduction kernels
    say(f"verify one expert {shape.name} T={T}")
    w13, w2 = synth.expert_f16(shape, 0, 0)
    x = synth.tokens(shape, T, step=7)
    ref = oracle.expert_ffn_f16(x, w13, w2)
    from gpu_util import upload_f16
    tab, keep = upload_f16([(w13, w2)])
    iota = torch.arange(T, dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    ws = fve.new_workspace(1, T, 1, shape.H, shape.I, 1)
    y = fve.verify_grouped_gemm(dev(x), iota, offs, tab, T, T, shape.H, shape.I, 1, ws)
    st = assert_fp16_close(host(y)[:T], ref, f"verify one expert {shape.name} T={T}")
    say(f"  l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")
