"""GPU parity of moe_draft_layer, the one-launch one-token draft layer
([S1] Key Contributions 4: routing and expert sub-computations of a draft
step inside a single launch).  Every output must be bit-identical to the
split path it fuses -- moe_draft_route_ffn, then moe_combine with the norm
epilogue and moe_combine_route_logits for the next layer's logits -- and the
layer output must match the oracle's moe_layer within the FP16 bars.  Calls
repeat on one workspace (the grid barriers' counters return to zero after
every call) with changing tokens, so stale values from an earlier call would
show."""
import dataclasses

import numpy as np
import pytest
import torch

import fp16_verify_expert_amd as fve
import oracle
import synth
from gpu_util import Layer, assert_fp16_close, dev, host, say

pytestmark = pytest.mark.gpu

# the instantiated geometries: Phi-3.5-MoE (no shared expert), DeepSeek-V2-Lite
# (two ungated shared experts as one of I = 2816), Qwen1.5-MoE (gated shared
# expert of I = 5632), and the H 2048 / I 1408 routed experts alone
_DS_NOSH = dataclasses.replace(synth.DS, name="ds_routed_only", shared_I=0)
CASES = [(synth.PHI, (0, 3, 7)), (synth.DS, (1, 5)), (synth.QWEN, (2, 6)), (_DS_NOSH, (4,))]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    fve.lib()
    torch.cuda.init()


def _err():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def _split(L, shape, dx, res, nxt, counters, logits=None):
    """The split path: moe_draft_route_ffn, then the combine with the norm
    epilogue and the next layer's logits."""
    E, k, H, I = shape.E, shape.k, shape.H, shape.I
    ws = fve.new_workspace(0, 1, k, H, I, E)
    sh = None if L.shared is None else (dev(L.shared["w13"]), dev(L.shared["w2"]))
    r = fve.moe_draft_route_ffn(dx, L.d_router, k, L.t4, I, ws, shape.renormalize, L.d_gate,
                                counters=counters, layer=1, shared=sh, logits=logits)
    ids, w, gate, m, y = r[:5]
    so = r[5] if sh is not None else None
    out, xn, lg = fve.moe_combine_route_logits(y, m["pair_pos"], w, nxt[0], so, gate, res,
                                               nxt[1])
    return dict(topk_ids=ids, topk_w=w, shared_gate=gate, maps=m, y_sorted=y, shared_out=so,
                out=out, norm_out=xn, next_logits=lg)


def _fused(L, shape, dx, res, nxt, counters, ws, logits=None, err=None):
    E, k, I = shape.E, shape.k, shape.I
    sh = None if L.shared is None else (dev(L.shared["w13"]), dev(L.shared["w2"]))
    return fve.moe_draft_layer(dx, L.d_router, k, L.t4, I, ws, shape.renormalize, L.d_gate,
                               logits=logits, counters=counters, layer=1, err_word=err,
                               shared=sh, residual=res, norm_out=True, next_router=nxt[0],
                               next_shared_gate=nxt[1])


def _same(a, b, k, what):
    for key in ("topk_ids", "topk_w", "out", "norm_out", "next_logits"):
        assert torch.equal(a[key], b[key]), f"{what}: {key}"
    if a["shared_gate"] is not None:
        assert torch.equal(a["shared_gate"], b["shared_gate"]), f"{what}: shared_gate"
    if a["shared_out"] is not None:
        assert torch.equal(a["shared_out"], b["shared_out"]), f"{what}: shared_out"
    assert torch.equal(a["y_sorted"][:k], b["y_sorted"][:k]), f"{what}: y_sorted"
    for key in ("offsets", "active", "n_active"):
        assert torch.equal(a["maps"][key], b["maps"][key]), f"{what}: {key}"
    for key in ("sorted_token", "sorted_pair", "pair_pos"):
        assert torch.equal(a["maps"][key][:k], b["maps"][key][:k]), f"{what}: {key}"


def _next(shape):
    wr = synth.router(shape, 1)
    sh = synth.shared_expert(shape, 1)
    g = None if sh is None or sh.get("gate") is None else sh["gate"]
    return (dev(wr), None if g is None else dev(g))


@pytest.mark.parametrize("shape,steps", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_draft_layer_matches_split_path_and_oracle(shape, steps):
    say(f"draft layer {shape.name} steps={steps}")
    E, k, H, I = shape.E, shape.k, shape.H, shape.I
    if not fve.draft_layer_supported(H, I, E, k, shape.shared_I):
        pytest.fail(f"no one-launch geometry for {shape.name}")
    xs = [synth.tokens(shape, 1, step=s) for s in steps]
    L = Layer(shape, xs, int4=True, f16=False)
    nxt = _next(shape)
    ws = fve.new_layer_workspace(k, H, I, E)
    err = _err()
    c0 = np.random.default_rng(7).integers(0, 50, size=(2, E)).astype(np.int32)
    c_split, c_fused = dev(c0), dev(c0)
    refs = []
    for j, x in enumerate(xs):
        dx = dev(x)
        res = dev(synth.tokens(shape, 1, step=100 + steps[j]))
        a = _split(L, shape, dx, res, nxt, c_split)
        torch.cuda.synchronize()
        refs.append((dx, res, {kk: (v.clone() if torch.is_tensor(v) else
                                    (None if v is None else {q: t.clone() for q, t in v.items()}))
                               for kk, v in a.items()}))
    # every token twice, interleaved, on one workspace: no state survives a call
    order = list(range(len(xs))) * 2
    for n, j in enumerate(order):
        dx, res, a = refs[j]
        b = _fused(L, shape, dx, res, nxt, c_fused, ws, err=err)
        torch.cuda.synchronize()
        assert int(host(err)[0]) == 0, f"device error word {int(host(err)[0])}"
        _same(a, b, k, f"{shape.name} call {n} (token {j})")
        assert not ws[:8].any(), "barrier counters not returned to zero"
    # the split path counted each token once, the fused path twice
    assert np.array_equal(host(c_fused) - c0, 2 * (host(c_split) - c0))
    # logits from the launch before (the chained form): the same bits
    dx, res, a = refs[0]
    lg = oracle.logits_pinned_f32(host(dx), L.router)[0]
    if L.d_gate is not None:
        lg = np.concatenate([lg, oracle.logits_pinned_f32(host(dx), L.shared["gate"][None])[0]])
    b = _fused(L, shape, dx, res, nxt, None, ws, logits=dev(lg.astype(np.float32)), err=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    _same(a, b, k, f"{shape.name} with logits")
    # the oracle: the layer output (residual block) and the next logits
    x0 = host(dx)
    ref = oracle.moe_layer(x0, L.router, k, L.int4, "int4", shared=L.shared,
                           renormalize=shape.renormalize, residual=host(res))
    assert np.array_equal(host(b["topk_ids"]), ref["route"]["ids"])
    st = assert_fp16_close(host(b["out"]), ref["out"], f"draft layer {shape.name}")
    say(f"  out l2={st['l2']:.2e} maxabs={st['maxabs']:.2e}")
    lg_next = oracle.logits_pinned_f32(host(b["norm_out"]), host(nxt[0]))[0]
    assert np.array_equal(host(b["next_logits"])[:E], lg_next.astype(np.float32))


def test_draft_layer_without_norm_or_residual():
    """The plain layer (no residual, no norm epilogue, no next router): out
    bit-identical to moe_draft_route_ffn + moe_combine."""
    s = synth.PHI
    x = synth.tokens(s, 1, step=11)
    L = Layer(s, [x], int4=True, f16=False)
    dx = dev(x)
    ws0 = fve.new_workspace(0, 1, s.k, s.H, s.I, s.E)
    ids, w, gate, m, y = fve.moe_draft_route_ffn(dx, L.d_router, s.k, L.t4, s.I, ws0)
    out = fve.moe_combine(y, m["pair_pos"], w)
    ws = fve.new_layer_workspace(s.k, s.H, s.I, s.E)
    b = fve.moe_draft_layer(dx, L.d_router, s.k, L.t4, s.I, ws)
    torch.cuda.synchronize()
    assert torch.equal(b["out"], out)
    assert torch.equal(b["topk_ids"], ids) and torch.equal(b["y_sorted"][:s.k], y[:s.k])
    assert b["norm_out"] is None and b["next_logits"] is None


def test_draft_layer_unsupported_shape_raises():
    """A shape without a one-launch geometry is refused before anything is
    enqueued (callers use the split path)."""
    s = synth.TINY
    assert not fve.draft_layer_supported(s.H, s.I, s.E, s.k, s.shared_I)
    x = synth.tokens(s, 1, step=0)
    L = Layer(s, [x], int4=True, f16=False)
    ws = fve.new_layer_workspace(s.k, s.H, s.I, s.E)
    with pytest.raises(fve.SmoeError) as ei:
        fve.moe_draft_layer(dev(x), L.d_router, s.k, L.t4, s.I, ws)
    assert ei.value.status == 3
