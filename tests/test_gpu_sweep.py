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
from hypothesis import HealthCheck, given, settings
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
