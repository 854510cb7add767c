"""w4a16_grouped_ffn_noalloc (the library's own scratch in place of a caller
workspace) against w4a16_grouped_ffn on the same inputs, through the C ABI:
two calls in a row on one GPU, the second with a smaller input, each equal
bit for bit to the workspace entry point and within the fp16 bars of the
oracle."""
import numpy as np
import pytest
import torch

import fp16_verify_expert_amd as fve
import oracle
import synth
from gpu_util import Layer, assert_fp16_close, dev, host, say

pytestmark = pytest.mark.gpu

# (shape, larger T, smaller T): the multi-row then the one-token kernels, and
# ragged multi-row groups then a few rows
SEQUENCES = [(synth.DS, 16, 1), (synth.TINY, 40, 3), (synth.PHI, 1, 1)]


def _run(L, x, T, err):
    s = L.shape
    dx = dev(x)
    ids, _, _ = fve.moe_route_topk(dx, L.d_router, s.k)
    maps = fve.moe_gather(ids, s.E, err)
    ws = fve.new_workspace(0, T, s.k, s.H, s.I, s.E)
    y_ws = fve.w4a16_grouped_ffn(dx, maps, L.t4, T, s.k, s.H, s.I, s.E, ws, err_word=err)
    y_na = torch.full_like(y_ws, float("nan"))
    fve.w4a16_grouped_ffn_noalloc(dx, maps, L.t4, T, s.k, s.H, s.I, s.E, y_sorted=y_na,
                                  err_word=err)
    return y_ws, y_na


@pytest.mark.parametrize("shape,T0,T1", SEQUENCES, ids=lambda v: getattr(v, "name", str(v)))
def test_noalloc_matches_workspace_entry_point(shape, T0, T1):
    xs = [synth.tokens(shape, T0, step=3), synth.tokens(shape, T1, step=4)]
    L = Layer(shape, xs, f16=False)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for T, x in zip((T0, T1), xs):
        say(f"noalloc {shape.name} T={T}")
        y_ws, y_na = _run(L, x, T, err)
        torch.cuda.synchronize()
        assert int(host(err)[0]) == 0
        rows = T * shape.k
        assert torch.equal(y_na[:rows], y_ws[:rows]), f"{shape.name} T={T}: outputs differ"
        r = oracle.route_topk(x, L.router, shape.k)
        ref = oracle.grouped_ffn(x, oracle.gather_maps(r["ids"], shape.E), L.int4, "int4")
        st = assert_fp16_close(host(y_na)[:rows], ref, f"noalloc {shape.name} T={T}")
        say(f"  bit-identical to the workspace call; l2={st['l2']:.2e}")


def test_noalloc_rejects_requests_beyond_the_scratch():
    s = synth.PHI
    T = 330                        # 660 rows of h at I = 6400: more than 4 MiB
    x = torch.zeros((T, s.H), dtype=torch.float16, device="cuda")
    maps = fve.moe_gather(torch.zeros((T, s.k), dtype=torch.int32, device="cuda"), s.E)
    table = fve.w4_expert_table([None] * s.E)
    with pytest.raises(fve.SmoeError) as ei:
        fve.w4a16_grouped_ffn_noalloc(x, maps, table, T, s.k, s.H, s.I, s.E)
    assert ei.value.status == 2 and "scratch" in str(ei.value)
