"""Randomised shapes through the whole layer on the GPU (hypothesis, fixed
derandomised examples): E <= 64, k <= min(E, 8), T <= 33, H and I in
128 * {1..4}.  For each drawn layer: routing ids and the gather maps exact
against the oracle, the INT4 draft FFN and the FP16 verify FFN within the
fp16 bars of the oracle's per-expert loop, and the layer output of both
kinds within the bars of oracle.moe_layer.  The first failing example stops
the sweep (hypothesis shrinks it and reports it)."""
import dataclasses

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, example, given, settings
from hypothesis import strategies as st

import fp16_verify_expert_amd as fve
import oracle
import synth
from gpu_util import Layer, assert_fp16_close, dev, host, run_layer, say

pytestmark = pytest.mark.gpu


@st.composite
def layer_shapes(draw):
    E = draw(st.integers(1, 64))
    k = draw(st.integers(1, min(E, 8)))
    T = draw(st.integers(1, 33))
    H = 128 * draw(st.integers(1, 4))
    I = 128 * draw(st.integers(1, 4))
    return E, k, T, H, I


@settings(max_examples=24, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(layer_shapes())
def test_random_layer_shapes(shape):
    E, k, T, H, I = shape
    say(f"sweep E={E} k={k} T={T} H={H} I={I}")
    s = dataclasses.replace(synth.TINY, name=f"sweep_{E}_{k}_{H}_{I}", E=E, k=k, H=H, I=I)
    x = synth.tokens(s, T, step=E + 7 * k + T)
    L = Layer(s, [x])
    dx = dev(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    r = oracle.route_topk(x, L.router, k)
    maps = oracle.gather_maps(r["ids"], E)
    for kind, experts in (("int4", L.int4), ("f16", L.f16)):
        got = run_layer(L, dx, kind, err)
        torch.cuda.synchronize()
        assert int(host(err)[0]) == 0
        assert np.array_equal(host(got["ids"]), r["ids"])
        for key in ("offsets", "active", "n_active"):
            assert np.array_equal(host(got["maps"][key]).ravel(), np.ravel(maps[key])), key
        rows = T * k
        for key in ("sorted_token", "sorted_pair", "pair_pos"):
            assert np.array_equal(host(got["maps"][key])[:rows], maps[key][:rows]), key
        y_ref = oracle.grouped_ffn(x, maps, experts, kind)
        assert_fp16_close(host(got["y"])[:rows], y_ref, f"{kind} FFN {shape}")
        ref = oracle.moe_layer(x, L.router, k, experts, kind)
        assert_fp16_close(host(got["out"]), ref["out"], f"{kind} layer {shape}")


@st.composite
def shared_layer_shapes(draw):
    E = draw(st.integers(1, 64))
    k = draw(st.integers(1, min(E, 8)))
    T = draw(st.sampled_from([1, 1, 2, 3, 4, 5, 8, 9, 16, 17, 33]))
    H = draw(st.sampled_from([128, 256, 512, 1024, 2048]))
    I = 128 * draw(st.integers(1, 4))
    Is = 128 * draw(st.integers(1, 12))
    gated = draw(st.booleans())
    return E, k, T, H, I, Is, gated


@settings(max_examples=20, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(shared_layer_shapes())
# branches the draws may miss: MFMA shared items (5-16 rows, hidden and
# shared intermediate >= 1024), one-token steps with the shared columns fused
# into both launches (DeepSeek- and Qwen-like chunk counts), few-row
# matrix-vector items
@example((16, 4, 9, 1024, 256, 1024, True))
@example((8, 2, 5, 1024, 128, 1152, False))
@example((16, 2, 16, 2048, 256, 1536, True))
@example((64, 6, 1, 2048, 256, 2816, False))
@example((60, 4, 1, 2048, 128, 5632, True))
@example((8, 2, 4, 2048, 128, 1024, True))
def test_random_shared_expert_layers(shape):
    """Randomised layers with a dense shared expert (gated or not) through the
    fused entry points, whose launch forms depend on the shape: the one-token
    draft step (moe_draft_route_ffn: the shared columns inside its launches
    where their chunk counts allow, else launches of their own), the
    multi-row draft (w4a16_grouped_ffn_shared: matrix-vector or MFMA shared
    items, or separate launches) and the verify (verify_grouped_gemm_shared).
    Routing and maps exact, layer outputs within the fp16 bars of
    oracle.moe_layer with the shared term."""
    E, k, T, H, I, Is, gated = shape
    say(f"shared sweep E={E} k={k} T={T} H={H} I={I} Is={Is} gated={gated}")
    s = dataclasses.replace(synth.TINY, name=f"sw_{E}_{k}_{H}_{I}_{Is}_{int(gated)}", E=E, k=k,
                            H=H, I=I, shared_I=Is, shared_gate=gated)
    x = synth.tokens(s, T, step=E + 3 * k + T + Is // 128)
    L = Layer(s, [x])
    assert L.shared is not None and (L.d_gate is not None) == gated
    dx = dev(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sw = (dev(L.shared["w13"]), dev(L.shared["w2"]))
    r = oracle.route_topk(x, L.router, k, False, L.shared.get("gate"))
    maps = oracle.gather_maps(r["ids"], E)
    rows = T * k
    for kind, experts in (("int4", L.int4), ("f16", L.f16)):
        if kind == "int4" and T == 1:
            ws = fve.new_workspace(0, 1, k, H, I, E)
            ids, w, gate, gm, y, sh = fve.moe_draft_route_ffn(
                dx, L.d_router, k, L.t4, I, ws, False, L.d_gate, err_word=err, shared=sw)
        else:
            ids, w, gate = fve.moe_route_topk(dx, L.d_router, k, False, L.d_gate)
            gm = fve.moe_gather(ids, E, err)
            if kind == "int4":
                ws = fve.new_workspace(0, T, k, H, I, E)
                y, sh = fve.w4a16_grouped_ffn_shared(dx, gm, L.t4, T, k, H, I, E, ws, sw,
                                                     err_word=err)
            else:
                ws = fve.new_workspace(1, T, k, H, I, E)
                y, sh = fve.verify_grouped_gemm_shared(
                    dx, gm["sorted_token"], gm["offsets"], L.t16, T, rows, H, I, E, ws, sw,
                    active=gm["active"], n_active=gm["n_active"], err_word=err)
        out = fve.moe_combine(y, gm["pair_pos"], w, sh, gate)
        torch.cuda.synchronize()
        assert int(host(err)[0]) == 0
        assert np.array_equal(host(ids), r["ids"])
        for key in ("offsets", "active", "n_active"):
            assert np.array_equal(host(gm[key]).ravel(), np.ravel(maps[key])), key
        for key in ("sorted_token", "sorted_pair", "pair_pos"):
            assert np.array_equal(host(gm[key])[:rows], maps[key][:rows]), key
        ref = oracle.moe_layer(x, L.router, k, experts, kind, shared=L.shared)
        assert_fp16_close(host(sh), ref["shared_out"], f"{kind} shared {shape}")
        assert_fp16_close(host(y)[:rows], ref["y_sorted"], f"{kind} FFN {shape}")
        assert_fp16_close(host(out), ref["out"], f"{kind} layer {shape}")


@st.composite
def dense_shapes(draw):
    E = draw(st.integers(1, 12))
    k = draw(st.integers(1, min(E, 4)))
    per = draw(st.sampled_from([64, 100, 128, 160, 256, 300]))  # mean rows per expert
    T = max(1, (per * E + k - 1) // k)
    H = 128 * draw(st.integers(1, 4))
    I = 128 * draw(st.integers(1, 3))
    return E, k, T, H, I


@settings(max_examples=16, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(dense_shapes())
# the register-staged form (under a full row tile per expert), the ring form
# with 256- and 128-column down tiles (H a multiple of 256 or not)
@example((8, 2, 400, 256, 256))
@example((4, 2, 512, 512, 128))
@example((4, 2, 512, 384, 256))
def test_random_dense_regime(shape):
    """Randomised shapes in the dense regime of verify_grouped_gemm (at least
    64 rows per expert): the tiled GEMM in its register-staged or ring form,
    full and partial column blocks, against the oracle's per-expert loop."""
    E, k, T, H, I = shape
    say(f"dense sweep E={E} k={k} T={T} H={H} I={I}")
    s = dataclasses.replace(synth.TINY, name=f"dn_{E}_{k}_{H}_{I}", E=E, k=k, H=H, I=I)
    x = synth.tokens(s, T, step=3 * E + k)
    L = Layer(s, [x], int4=False)
    dx = dev(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    r = oracle.route_topk(x, L.router, k)
    maps = oracle.gather_maps(r["ids"], E)
    rows = T * k
    assert rows >= 64 * min(E, rows)
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, k)
    gm = fve.moe_gather(ids, E, err)
    ws = fve.new_workspace(1, T, k, H, I, E)
    y = fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], L.t16, T, rows, H, I, E,
                                ws, active=gm["active"], n_active=gm["n_active"], err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert np.array_equal(host(ids), r["ids"])
    ref = oracle.grouped_ffn(x, maps, L.f16, "f16")
    assert_fp16_close(host(y)[:rows], ref, f"dense {shape}")


@st.composite
def draft_format_shapes(draw):
    E = draw(st.integers(1, 64))
    k = draw(st.integers(1, min(E, 8)))
    T = draw(st.sampled_from([1, 1, 2, 3, 4, 7, 16, 17, 33]))
    H = 128 * draw(st.integers(1, 6))
    I = 128 * draw(st.integers(1, 6))
    fmt = draw(st.sampled_from(["int2", "int4", "int8", "awq"]))
    return E, k, T, H, I, fmt


@settings(max_examples=20, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(draft_format_shapes())
@example((16, 2, 1, 1024, 1024, "int8"))   # long 8-bit reductions at one token
@example((16, 4, 16, 1024, 512, "int2"))
@example((8, 2, 5, 512, 384, "awq"))
def test_random_draft_formats(shape):
    """Randomised shapes for the other draft formats: wq_grouped_ffn at 2, 4
    and 8 bits (GPTQ layout) and awq_grouped_ffn (per-input-channel divisors)
    against the oracle's per-expert loop of the same codes."""
    E, k, T, H, I, fmt = shape
    say(f"format sweep {fmt} E={E} k={k} T={T} H={H} I={I}")
    s = dataclasses.replace(synth.TINY, name=f"fm_{E}_{k}_{H}_{I}", E=E, k=k, H=H, I=I)
    x = synth.tokens(s, T, step=2 * E + k + T)
    router = synth.router(s)
    r = oracle.route_topk(x, router, k)
    touched = sorted(set(int(e) for e in r["ids"].ravel()))
    ex = [None] * E
    for e in touched:
        w13, w2 = synth.expert_f16(s, 0, e)
        ex[e] = (synth.expert_awq(s, 0, e, w13, w2) if fmt == "awq"
                 else synth.expert_int4(w13, w2, bits=int(fmt[3:])))
    gpu = [None if q is None else {key: tuple(dev(t) for t in q[key]) for key in ("w13", "w2")}
           for q in ex]
    table = fve.w4_expert_table(gpu)
    maps = oracle.gather_maps(r["ids"], E)
    ref = oracle.grouped_ffn(x, maps, ex, fmt)
    dx = dev(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids, _, _ = fve.moe_route_topk(dx, dev(router), k)
    gm = fve.moe_gather(ids, E, err)
    ws = fve.new_workspace(0, T, k, H, I, E)
    if fmt == "awq":
        sc = [None if q is None else (dev(q["a13"]), dev(q["a2"])) for q in ex]
        stab = fve.awq_scale_table(sc)
        y = fve.awq_grouped_ffn(dx, gm, table, stab, T, k, H, I, E, ws, err_word=err)
    else:
        y = fve.wq_grouped_ffn(dx, gm, table, T, k, H, I, E, ws, int(fmt[3:]), err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert np.array_equal(host(ids), r["ids"])
    rows = T * k
    assert_fp16_close(host(y)[:rows], ref, f"{fmt} FFN {shape}")


@st.composite
def routing_shapes(draw):
    E = draw(st.sampled_from([1, 2, 7, 16, 60, 64, 100, 128, 256]))
    k = draw(st.integers(1, min(E, 16)))
    T = draw(st.sampled_from([1, 2, 5, 16, 33, 100, 257]))
    H = 128 * draw(st.integers(1, 16))
    renorm = draw(st.booleans())
    gated = draw(st.booleans())
    return E, k, T, H, renorm, gated


@settings(max_examples=24, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(routing_shapes())
@example((256, 16, 15, 2048, False, True))    # the largest router, spread plan
@example((256, 16, 257, 2048, False, True))   # beyond the plan's step size: refused
@example((64, 6, 16, 2048, False, False))     # DeepSeek-like, two-launch plan
@example((16, 2, 1, 4096, True, False))       # one token, renormalised
def test_random_routing(shape):
    """Randomised routing shapes through moe_route_topk and both forms of
    moe_route_plan (with a logits workspace: spread over the chip where the
    step is large; without: one workgroup or the routing kernel): ids, ELB
    counts (layer 1 of 2) and the gather maps exact, weights and the shared
    gate within 1e-5 of the oracle; steps above the plan's 1024 pairs or
    4096 logits are refused with a shape error."""
    E, k, T, H, renorm, gated = shape
    say(f"routing sweep E={E} k={k} T={T} H={H} renorm={renorm} gated={gated}")
    s = dataclasses.replace(synth.TINY, name=f"rt_{E}_{k}_{H}", E=E, k=k, H=H,
                            shared_I=128 if gated else 0, shared_gate=gated,
                            renormalize=renorm)
    router = synth.router(s)
    gate_vec = synth.shared_expert(s)["gate"] if gated else None
    x = synth.tokens(s, T, step=E + k + T)
    ref = oracle.route_topk(x, router, k, renorm, gate_vec)
    maps = oracle.gather_maps(ref["ids"], E)
    cref = oracle.elb_update(np.zeros((2, E), np.int32), ref["ids"], 1)
    dx, dr = dev(x), dev(router)
    dg = dev(gate_vec) if gated else None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def check(ids, w, gate, what):
        assert np.array_equal(host(ids), ref["ids"]), what
        assert np.allclose(host(w), ref["weights"], rtol=1e-5, atol=1e-7), what
        if gated:
            assert np.allclose(host(gate), ref["gate"], rtol=1e-5, atol=1e-7), what

    ids, w, gate = fve.moe_route_topk(dx, dr, k, renorm, dg)
    torch.cuda.synchronize()
    check(ids, w, gate, "moe_route_topk")
    rows = T * k
    for spread in (True, False):
        counters = torch.zeros((2, E), dtype=torch.int32, device="cuda")
        if rows > 1024 or T * (E + 1) > 4096:  # beyond the plan's documented sizes: refused
            with pytest.raises(fve.SmoeError):
                fve.moe_route_plan(dx, dr, k, renorm, dg, counters=counters, layer=1,
                                   err_word=err, spread=spread)
            continue
        ids, w, gate, gm = fve.moe_route_plan(dx, dr, k, renorm, dg, counters=counters, layer=1,
                                             err_word=err, spread=spread)
        torch.cuda.synchronize()
        assert int(host(err)[0]) == 0
        check(ids, w, gate, f"moe_route_plan spread={spread}")
        assert np.array_equal(host(counters), cref), f"ELB spread={spread}"
        for key in ("offsets", "active", "n_active"):
            assert np.array_equal(host(gm[key]).ravel(), np.ravel(maps[key])), (key, spread)
        for key in ("sorted_token", "sorted_pair", "pair_pos"):
            assert np.array_equal(host(gm[key])[:rows], maps[key][:rows]), (key, spread)


@st.composite
def one_token_shapes(draw):
    E = draw(st.sampled_from([1, 2, 8, 16, 60, 64, 100, 256]))
    k = draw(st.integers(1, min(E, 16)))
    H = 128 * draw(st.integers(1, 16))
    I = 128 * draw(st.integers(1, 12))
    renorm = draw(st.booleans())
    return E, k, H, I, renorm


@settings(max_examples=20, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(one_token_shapes())
@example((256, 16, 2048, 512, False))
@example((16, 2, 2048, 1536, True))
def test_random_one_token_draft(shape):
    """Randomised one-token draft steps through moe_draft_route_ffn (the
    routing folded into the gate/up launch; no shared expert) with ELB counts
    (layer 0 of 1) and moe_combine: ids, counts and maps exact, weights within
    1e-5, y and the layer output against oracle.moe_layer."""
    E, k, H, I, renorm = shape
    say(f"one-token sweep E={E} k={k} H={H} I={I} renorm={renorm}")
    s = dataclasses.replace(synth.TINY, name=f"ot_{E}_{k}_{H}_{I}", E=E, k=k, H=H, I=I,
                            renormalize=renorm)
    x = synth.tokens(s, 1, step=E + k + H // 128)
    L = Layer(s, [x], f16=False)
    dx = dev(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    counters = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    ws = fve.new_workspace(0, 1, k, H, I, E)
    ids, w, _, gm, y = fve.moe_draft_route_ffn(dx, L.d_router, k, L.t4, I, ws, renorm,
                                               counters=counters, err_word=err)
    out = fve.moe_combine(y, gm["pair_pos"], w)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    ref = oracle.moe_layer(x, L.router, k, L.int4, "int4", renormalize=renorm)
    assert np.array_equal(host(ids), ref["route"]["ids"])
    assert np.allclose(host(w), ref["route"]["weights"], rtol=1e-5, atol=1e-7)
    assert np.array_equal(host(counters),
                          oracle.elb_update(np.zeros((1, E), np.int32), ref["route"]["ids"], 0))
    for key in ("offsets", "active", "n_active"):
        assert np.array_equal(host(gm[key]).ravel(), np.ravel(ref["maps"][key])), key
    for key in ("sorted_token", "sorted_pair", "pair_pos"):
        assert np.array_equal(host(gm[key])[:k], ref["maps"][key][:k]), key
    assert_fp16_close(host(y)[:k], ref["y_sorted"], f"one-token FFN {shape}")
    assert_fp16_close(host(out), ref["out"], f"one-token layer {shape}")


@st.composite
def combine_shapes(draw):
    T = draw(st.sampled_from([1, 1, 2, 3, 8, 9, 17, 33, 100]))
    k = draw(st.integers(1, 16))
    H = 128 * draw(st.integers(1, 32))
    shared = draw(st.sampled_from(["none", "ungated", "gated"]))
    resid = draw(st.booleans())
    norm = draw(st.booleans())
    drop = draw(st.booleans())
    return T, k, H, shared, resid, norm, drop


@settings(max_examples=24, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(combine_shapes())
@example((1, 6, 2048, "none", True, True, False))
@example((1, 4, 2048, "gated", True, True, True))
@example((100, 8, 4096, "ungated", True, True, True))
def test_random_combine(shape):
    """Randomised combines: moe_combine (slots, dropped pairs, the shared term
    with or without its gate, the residual, the norm epilogue) against
    oracle.combine and oracle.rms_norm; for one token also
    moe_combine_route_logits, whose out and norm_out equal moe_combine's bit
    for bit and whose logits equal the oracle's pinned-order fp32 logits of
    that norm_out."""
    T, k, H, shared, resid, norm, drop = shape
    say(f"combine sweep T={T} k={k} H={H} shared={shared} resid={resid} norm={norm} drop={drop}")
    rng = np.random.default_rng(T * 1000 + k * 10 + H // 128)
    n = T * k
    y = rng.standard_normal((n, H)).astype(np.float16)
    pp = rng.permutation(n).astype(np.int32)
    if drop:
        pp[rng.integers(0, n)] = -1
    w = rng.random((T, k)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float16) if shared != "none" else None
    c = rng.random(T).astype(np.float32) if shared == "gated" else None
    res = rng.standard_normal((T, H)).astype(np.float16) if resid else None
    d = lambda a: None if a is None else dev(a)
    ref = oracle.combine(y, pp, w.astype(np.float64), sh, c, res)
    got = fve.moe_combine(dev(y), dev(pp), dev(w), d(sh), d(c), d(res), norm_out=norm)
    out = got[0] if norm else got
    torch.cuda.synchronize()
    assert_fp16_close(host(out), ref, f"combine {shape}", l2=1e-3, maxabs=4e-3)
    if norm:
        assert_fp16_close(host(got[1]), oracle.rms_norm(host(out)), f"combine norm {shape}",
                          l2=1e-3, maxabs=4e-3)
    if T == 1:
        E = 1 + (k * 7) % 64
        rs = dataclasses.replace(synth.TINY, name=f"cb_{E}_{H}", E=E, H=H)
        router = synth.router(rs, 3)
        wsg = rng.standard_normal(H).astype(np.float16) if shared == "gated" else None
        o2, n2, lg = fve.moe_combine_route_logits(dev(y), dev(pp), dev(w), dev(router), d(sh),
                                                  d(c), d(res), d(wsg))
        o1, n1 = fve.moe_combine(dev(y), dev(pp), dev(w), d(sh), d(c), d(res), norm_out=True)
        torch.cuda.synchronize()
        assert torch.equal(o2, o1) and torch.equal(n2, n1)
        ref_lg = oracle.logits_pinned_f32(host(n1), router)[0]
        assert np.array_equal(host(lg)[:E].view(np.uint32), ref_lg.view(np.uint32))
        if wsg is not None:
            ref_g = oracle.logits_pinned_f32(host(n1), wsg[None, :])[0]
            assert np.array_equal(host(lg)[E:].view(np.uint32), ref_g.view(np.uint32))


@st.composite
def mask_shapes(draw):
    E = draw(st.integers(2, 64))
    k = draw(st.integers(1, min(E, 8)))
    T = draw(st.sampled_from([1, 2, 4, 9, 17, 33, 200]))
    H = 128 * draw(st.integers(1, 16))
    I = 128 * draw(st.integers(1, 12))
    frac = draw(st.sampled_from([0.0, 0.25, 0.5, 1.0]))
    return E, k, T, H, I, frac


@settings(max_examples=20, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(mask_shapes())
@example((16, 2, 17, 2048, 1024, 0.5))    # ring kernels at K+1 = 17
@example((8, 2, 200, 256, 256, 0.25))     # dense regime
@example((60, 4, 9, 2048, 1408, 0.5))     # 2-wave ring, Qwen-like
def test_random_verify_mask(shape):
    """verify_grouped_gemm over a random expert mask and then its complement
    into the same output (hits computed before the staged misses arrive)
    equals one call over all experts bit for bit, in every launch form the
    shapes reach (matrix-vector, register, ring and dense regimes)."""
    E, k, T, H, I, frac = shape
    say(f"mask sweep E={E} k={k} T={T} H={H} I={I} frac={frac}")
    s = dataclasses.replace(synth.TINY, name=f"mk_{E}_{k}_{H}_{I}", E=E, k=k, H=H, I=I)
    x = synth.tokens(s, T, step=5 * E + k + T)
    L = Layer(s, [x], int4=False)
    dx = dev(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, k)
    gm = fve.moe_gather(ids, E, err)
    rows = T * k
    ws = fve.new_workspace(1, T, k, H, I, E)
    full = fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], L.t16, T, rows, H, I,
                                   E, ws, active=gm["active"], n_active=gm["n_active"],
                                   err_word=err)
    rng = np.random.default_rng(E * 100 + T)
    hit = torch.from_numpy((rng.random(E) < frac).astype(np.uint8)).cuda()
    y = torch.full_like(full, float("nan"))
    for m in (hit, 1 - hit):
        fve.verify_grouped_gemm(dx, gm["sorted_token"], gm["offsets"], L.t16, T, rows, H, I, E,
                                ws, active=gm["active"], n_active=gm["n_active"],
                                expert_mask=m, y_sorted=y, err_word=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert torch.equal(y[:rows], full[:rows])
